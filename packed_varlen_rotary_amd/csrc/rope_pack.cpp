// Host-side Best-Fit-Decreasing packing and the packed-metadata cache
// (contract in include/rope_pack.h).
//
// Sources: "Chronicals: A High-Performance Framework for LLM Fine-Tuning with
// 3.51x Speedup over Unsloth", abstract, optimisation (4) (Best-Fit Decreasing
// packing); "Unsloth und NVIDIA optimieren LLM-Training um zusätzliche 25%"
// (lumeric.app), item (1) (caching packed-sequence metadata to avoid repeated
// GPU-CPU synchronisations).
//
// Packing is O(n log n): the open bins sit in an ordered set keyed by
// (remaining room, bin index), so the best fit of a length is the set's
// lower bound of (length, 0), which also breaks equal rooms towards the bin
// opened first.  The cache keys a batch by (capacity, lengths) with a 64-bit
// FNV-1a hash and compares the stored lengths exactly; plans sit in an LRU
// list.  A hit touches no device state.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <list>
#include <mutex>
#include <numeric>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "rope_pack.h"
#include "rope_qk.h"

namespace {

constexpr int64_t kMaxTokens = INT32_MAX;

int check_lengths(const int32_t* lengths, int64_t n, int64_t capacity) {
  if (n < 0 || capacity < 1 || capacity > kMaxTokens) return ROPE_QK_ERR_SHAPE;
  if (n > 0 && lengths == nullptr) return ROPE_QK_ERR_NULL;
  for (int64_t i = 0; i < n; ++i)
    if (lengths[i] < 0 || lengths[i] > capacity) return ROPE_QK_ERR_SHAPE;
  return ROPE_QK_OK;
}

// Best-Fit-Decreasing into bin_of / offset_of (lengths already checked).
int64_t bfd(const int32_t* lengths, int64_t n, int64_t capacity, int32_t* bin_of, int32_t* offset_of) {
  std::vector<int64_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), int64_t(0));
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return lengths[a] > lengths[b]; });
  std::set<std::pair<int64_t, int64_t>> open;  // (room, bin)
  int64_t nbins = 0;
  for (const int64_t i : order) {
    const int64_t need = lengths[i];
    auto it = open.lower_bound({need, int64_t(0)});
    int64_t bin, room;
    if (it == open.end()) {
      bin = nbins++;
      room = capacity;
    } else {
      bin = it->second;
      room = it->first;
      open.erase(it);
    }
    bin_of[i] = static_cast<int32_t>(bin);
    offset_of[i] = static_cast<int32_t>(capacity - room);
    open.insert({room - need, bin});
  }
  return nbins;
}

// cu_seqlens of a placement; ROPE_QK_ERR_SHAPE if a bin's sequences do not
// tile it from token 0.
int build_cu(const int32_t* lengths, const int32_t* bin_of, const int32_t* offset_of, int64_t n, int64_t nbins,
             int64_t capacity, int32_t* cu_out, int64_t* nseg) {
  if (nbins < 0 || nbins * capacity > kMaxTokens) return ROPE_QK_ERR_SHAPE;
  // items ordered by (bin, offset), equal offsets (zero lengths first) by length
  std::vector<int64_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), int64_t(0));
  for (int64_t i = 0; i < n; ++i)
    if (bin_of[i] < 0 || bin_of[i] >= nbins || offset_of[i] < 0) return ROPE_QK_ERR_SHAPE;
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (bin_of[a] != bin_of[b]) return bin_of[a] < bin_of[b];
    if (offset_of[a] != offset_of[b]) return offset_of[a] < offset_of[b];
    if (lengths[a] != lengths[b]) return lengths[a] < lengths[b];
    return a < b;
  });
  int64_t k = 0, s = 0;
  cu_out[s++] = 0;
  for (int64_t b = 0; b < nbins; ++b) {
    int64_t pos = b * capacity;
    for (; k < n && bin_of[order[k]] == b; ++k) {
      const int64_t i = order[k];
      if (b * capacity + offset_of[i] != pos) return ROPE_QK_ERR_SHAPE;
      pos += lengths[i];
      if (pos > (b + 1) * capacity) return ROPE_QK_ERR_SHAPE;
      cu_out[s++] = static_cast<int32_t>(pos);
    }
    if (pos < (b + 1) * capacity) cu_out[s++] = static_cast<int32_t>((b + 1) * capacity);
  }
  *nseg = s - 1;
  return ROPE_QK_OK;
}

uint64_t fnv1a(const int32_t* lengths, int64_t n, int64_t capacity) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t v) {
    for (int byte = 0; byte < 8; ++byte) {
      h ^= (v >> (8 * byte)) & 0xFFu;
      h *= 1099511628211ull;
    }
  };
  mix(static_cast<uint64_t>(capacity));
  mix(static_cast<uint64_t>(n));
  for (int64_t i = 0; i < n; ++i) mix(static_cast<uint32_t>(lengths[i]));
  return h;
}

struct Entry {
  uint64_t hash = 0;
  int64_t capacity = 0;
  std::vector<int32_t> lengths, bin_of, offset_of;
  int32_t* cu_host = nullptr;  // pinned when the cache has a device
  int32_t* cu_dev = nullptr;
  std::vector<int32_t> cu_pageable;  // host-only caches
  int64_t nseg = 0, nbins = 0;
  int32_t max_seqlen = 0;
};

// Makes `device` current for its lifetime (device >= 0) and restores the
// caller's current device afterwards.
struct DeviceScope {
  int prev = -1;
  bool ok = true;
  explicit DeviceScope(int device) {
    if (device < 0) return;
    ok = hipGetDevice(&prev) == hipSuccess && hipSetDevice(device) == hipSuccess;
  }
  ~DeviceScope() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

void release(Entry& e) {
  if (e.cu_dev != nullptr) (void)hipFree(e.cu_dev);
  if (e.cu_host != nullptr) (void)hipHostFree(e.cu_host);
  e.cu_dev = nullptr;
  e.cu_host = nullptr;
}

}  // namespace

struct rope_pack_cache {
  int64_t max_entries = 1;
  int device = -1;
  std::mutex mu;
  std::list<Entry> lru;  // most recently used first
  std::unordered_multimap<uint64_t, std::list<Entry>::iterator> index;
  int64_t hits = 0, misses = 0;
};

extern "C" {

int rope_pack_bfd(const int32_t* lengths, int64_t n, int64_t capacity, int32_t* bin_of, int32_t* offset_of,
                  int64_t* nbins) {
  if (nbins == nullptr) return ROPE_QK_ERR_NULL;
  const int status = check_lengths(lengths, n, capacity);
  if (status != ROPE_QK_OK) return status;
  if (n > 0 && (bin_of == nullptr || offset_of == nullptr)) return ROPE_QK_ERR_NULL;
  *nbins = bfd(lengths, n, capacity, bin_of, offset_of);
  return ROPE_QK_OK;
}

int rope_pack_cu_seqlens(const int32_t* lengths, const int32_t* bin_of, const int32_t* offset_of, int64_t n,
                         int64_t nbins, int64_t capacity, int32_t* cu_out, int64_t* nseg) {
  if (cu_out == nullptr || nseg == nullptr) return ROPE_QK_ERR_NULL;
  const int status = check_lengths(lengths, n, capacity);
  if (status != ROPE_QK_OK) return status;
  if (n > 0 && (bin_of == nullptr || offset_of == nullptr)) return ROPE_QK_ERR_NULL;
  return build_cu(lengths, bin_of, offset_of, n, nbins, capacity, cu_out, nseg);
}

int rope_pack_cache_create(int64_t max_entries, int device, rope_pack_cache** out) {
  if (out == nullptr) return ROPE_QK_ERR_NULL;
  if (max_entries < 1 || device < -1) return ROPE_QK_ERR_SHAPE;
  rope_pack_cache* c = new rope_pack_cache;
  c->max_entries = max_entries;
  c->device = device;
  *out = c;
  return ROPE_QK_OK;
}

int rope_pack_cache_get(rope_pack_cache* cache, const int32_t* lengths, int64_t n, int64_t capacity, void* stream,
                        rope_pack_plan* out) {
  if (cache == nullptr || out == nullptr) return ROPE_QK_ERR_NULL;
  int status = check_lengths(lengths, n, capacity);
  if (status != ROPE_QK_OK) return status;
  const uint64_t h = fnv1a(lengths, n, capacity);
  std::lock_guard<std::mutex> lock(cache->mu);
  std::list<Entry>::iterator found = cache->lru.end();
  auto range = cache->index.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const Entry& e = *it->second;
    if (e.capacity == capacity && static_cast<int64_t>(e.lengths.size()) == n &&
        std::equal(e.lengths.begin(), e.lengths.end(), lengths)) {
      found = it->second;
      break;
    }
  }
  int hit = 1;
  if (found != cache->lru.end()) {
    cache->lru.splice(cache->lru.begin(), cache->lru, found);  // most recently used
    ++cache->hits;
  } else {
    hit = 0;
    Entry e;
    e.hash = h;
    e.capacity = capacity;
    e.lengths.assign(lengths, lengths + n);
    e.bin_of.resize(static_cast<size_t>(n));
    e.offset_of.resize(static_cast<size_t>(n));
    e.nbins = bfd(lengths, n, capacity, e.bin_of.data(), e.offset_of.data());
    if (e.nbins * capacity > kMaxTokens) return ROPE_QK_ERR_SHAPE;
    const size_t cu_len = static_cast<size_t>(n + e.nbins + 1);
    int32_t* cu = nullptr;
    DeviceScope scope(cache->device);  // the cache's device while allocating; the caller's afterwards
    if (cache->device >= 0) {
      if (!scope.ok) return ROPE_QK_ERR_LAUNCH;
      if (hipHostMalloc(reinterpret_cast<void**>(&e.cu_host), cu_len * sizeof(int32_t)) != hipSuccess)
        return ROPE_QK_ERR_LAUNCH;
      cu = e.cu_host;
    } else {
      e.cu_pageable.resize(cu_len);
      cu = e.cu_pageable.data();
    }
    status = build_cu(lengths, e.bin_of.data(), e.offset_of.data(), n, e.nbins, capacity, cu, &e.nseg);
    if (status != ROPE_QK_OK) {
      release(e);
      return status;
    }
    int32_t longest = 0;
    for (int64_t s = 0; s < e.nseg; ++s) longest = std::max(longest, cu[s + 1] - cu[s]);
    e.max_seqlen = longest;
    if (cache->device >= 0) {
      const size_t bytes = static_cast<size_t>(e.nseg + 1) * sizeof(int32_t);
      if (hipMalloc(reinterpret_cast<void**>(&e.cu_dev), bytes) != hipSuccess ||
          hipMemcpyAsync(e.cu_dev, e.cu_host, bytes, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) !=
              hipSuccess) {
        release(e);
        return ROPE_QK_ERR_LAUNCH;
      }
    }
    // make room: evict least recently used plans
    while (static_cast<int64_t>(cache->lru.size()) >= cache->max_entries) {
      Entry& victim = cache->lru.back();
      auto vr = cache->index.equal_range(victim.hash);
      for (auto it = vr.first; it != vr.second; ++it) {
        if (&*it->second == &victim) {
          cache->index.erase(it);
          break;
        }
      }
      release(victim);
      cache->lru.pop_back();
    }
    cache->lru.push_front(std::move(e));
    cache->index.emplace(h, cache->lru.begin());
    found = cache->lru.begin();
    ++cache->misses;
  }
  const Entry& e = *found;
  out->cu_seqlens_device = e.cu_dev;
  out->cu_seqlens_host = e.cu_host != nullptr ? e.cu_host : e.cu_pageable.data();
  out->bin_of = e.bin_of.data();
  out->offset_of = e.offset_of.data();
  out->n = static_cast<int64_t>(e.lengths.size());
  out->nseg = e.nseg;
  out->nbins = e.nbins;
  out->T = e.nbins * e.capacity;
  out->max_seqlen = e.max_seqlen;
  out->hit = hit;
  return ROPE_QK_OK;
}

int rope_pack_cache_stats(const rope_pack_cache* cache, int64_t* hits, int64_t* misses, int64_t* entries) {
  if (cache == nullptr) return ROPE_QK_ERR_NULL;
  rope_pack_cache* c = const_cast<rope_pack_cache*>(cache);
  std::lock_guard<std::mutex> lock(c->mu);
  if (hits != nullptr) *hits = c->hits;
  if (misses != nullptr) *misses = c->misses;
  if (entries != nullptr) *entries = static_cast<int64_t>(c->lru.size());
  return ROPE_QK_OK;
}

void rope_pack_cache_destroy(rope_pack_cache* cache) {
  if (cache == nullptr) return;
  for (Entry& e : cache->lru) release(e);
  delete cache;
}

}  // extern "C"
