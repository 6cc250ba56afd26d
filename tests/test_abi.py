"""The C-ABI library: it loads, exports what include/rope_qk.h declares, and
its host-side argument checks return the documented status codes.

Everything here runs on the CPU: each call below is rejected (or is a no-op)
before the library makes any HIP call, so no pointer is dereferenced and no
kernel is launched.
"""

import ctypes
import os
import re
import subprocess

import pytest

import packed_varlen_rotary_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rope_qk.h")


def declared_functions():
    """Functions declared by every header under include/."""
    names = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", name)).read(), flags=re.S)
            names |= set(re.findall(r"\b(rope_\w+)\s*\(", text))
    return sorted(names)


def header_constants():
    consts = {}
    for m in re.finditer(r"#define\s+(ROPE_QK_\w+)\s+(-?\d+)", open(HEADER).read()):
        consts[m.group(1)] = int(m.group(2))
    return consts


C = header_constants()
lib = P.load()

# fake but 16-byte aligned device addresses; never dereferenced by these calls
# (1 TiB apart, so that the tensors of these calls never share memory)
Q, K, CU = 1 << 40, 2 << 40, 3 << 40


def fwd(q=Q, k=K, cu=CU, nseq=4, T=256, Hq=14, Hkv=2, D=64, qst=None, qsh=None, kst=None, ksh=None,
        theta=1e6, dtype=1, which="rope_qk_fwd"):
    qst = Hq * D if qst is None else qst
    qsh = D if qsh is None else qsh
    kst = Hkv * D if kst is None else kst
    ksh = D if ksh is None else ksh
    return getattr(lib, which)(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(cu), nseq, T, Hq, Hkv, D,
                               qst, qsh, kst, ksh, theta, dtype, None)


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(P.EXPORTS)


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(rope_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions())


def test_status_constants_match_binding():
    assert C["ROPE_QK_FP32"] == P.ROPE_QK_FP32 and C["ROPE_QK_BF16"] == P.ROPE_QK_BF16
    assert C["ROPE_QK_FP16"] == P.ROPE_QK_FP16
    for name, code in C.items():
        if "_ERR_" in name or name == "ROPE_QK_OK":
            s = P.rope_qk_strerror(code)
            assert s and s != "unknown status", name
    assert P.rope_qk_strerror(12345) == "unknown status"


@pytest.mark.parametrize("which", ["rope_qk_fwd", "rope_qk_bwd"])
def test_error_codes(which):
    f = lambda **kw: fwd(which=which, **kw)  # noqa: E731
    assert f(dtype=7) == C["ROPE_QK_ERR_DTYPE"]
    assert f(D=63) == C["ROPE_QK_ERR_SHAPE"]
    assert f(D=0) == C["ROPE_QK_ERR_SHAPE"]
    assert f(D=514) == C["ROPE_QK_ERR_SHAPE"]
    assert f(T=-1) == C["ROPE_QK_ERR_SHAPE"]
    assert f(nseq=-1) == C["ROPE_QK_ERR_SHAPE"]
    assert f(Hq=-2) == C["ROPE_QK_ERR_SHAPE"]
    assert f(T=2 ** 31) == C["ROPE_QK_ERR_SHAPE"]
    assert f(theta=0.0) == C["ROPE_QK_ERR_THETA"]
    assert f(theta=-1e4) == C["ROPE_QK_ERR_THETA"]
    assert f(theta=float("inf")) == C["ROPE_QK_ERR_THETA"]
    assert f(theta=float("nan")) == C["ROPE_QK_ERR_THETA"]
    assert f(q=0) == C["ROPE_QK_ERR_NULL"]
    assert f(k=0) == C["ROPE_QK_ERR_NULL"]
    assert f(cu=0) == C["ROPE_QK_ERR_NULL"]
    assert f(q=Q + 2) == C["ROPE_QK_ERR_ALIGN"]
    assert f(k=K + 8, dtype=0) == C["ROPE_QK_ERR_ALIGN"]
    assert f(D=72) == C["ROPE_QK_ERR_ALIGN"]  # (D/2)*2 bytes = 72, not a multiple of 16
    assert f(D=68, qst=14 * 68, kst=2 * 68, qsh=68, ksh=68, dtype=0) == C["ROPE_QK_ERR_ALIGN"]  # (D/2)*4 = 136 bytes
    assert f(qst=14 * 64 + 2, dtype=0) == C["ROPE_QK_ERR_ALIGN"]  # token stride of 8 bytes past 16
    assert f(qst=14 * 64 + 4) == C["ROPE_QK_ERR_ALIGN"]
    assert f(qsh=-64) == C["ROPE_QK_ERR_LAYOUT"]
    assert f(qsh=32) == C["ROPE_QK_ERR_LAYOUT"]  # heads overlap
    assert f(qst=64 * 13) == C["ROPE_QK_ERR_LAYOUT"]  # tokens overlap
    assert f(kst=64, ksh=64) == C["ROPE_QK_ERR_LAYOUT"]
    assert f(Hq=70000, Hkv=0, qst=70000 * 64) == C["ROPE_QK_ERR_SHAPE"]  # too many 16-byte chunks per token
    # fp16 shares bf16's 2-byte element checks
    assert f(D=72, dtype=2) == C["ROPE_QK_ERR_ALIGN"]
    assert f(q=Q + 8, dtype=2) == C["ROPE_QK_ERR_ALIGN"]
    assert f(qst=14 * 64 + 4, dtype=2) == C["ROPE_QK_ERR_ALIGN"]
    assert f(qsh=32, dtype=2) == C["ROPE_QK_ERR_LAYOUT"]
    assert f(dtype=3) == C["ROPE_QK_ERR_DTYPE"]


def test_no_ops_launch_nothing():
    # nothing to do: returns OK without touching the (fake) pointers or HIP
    assert fwd(T=0) == C["ROPE_QK_OK"]
    assert fwd(nseq=0) == C["ROPE_QK_OK"]
    assert fwd(Hq=0, Hkv=0) == C["ROPE_QK_OK"]
    assert fwd(T=0, q=0, k=0, cu=0) == C["ROPE_QK_OK"]
    # a tensor with no heads may be NULL; the checks of the other still apply
    assert fwd(Hkv=0, k=0, q=Q + 2) == C["ROPE_QK_ERR_ALIGN"]


def test_layouts_that_are_accepted_by_the_checks():
    # fused-QKV views (token stride > heads*D) and head-major layouts are not overlaps;
    # use an invalid dtype afterwards to stop before any launch: the layout check runs first
    # only when the dtype is valid, so instead check via a NULL cu with a valid layout
    assert fwd(qst=48 * 128, qsh=128, kst=48 * 128, ksh=128, D=128, Hq=32, Hkv=8, cu=0) == C["ROPE_QK_ERR_NULL"]
    assert fwd(qst=64, qsh=64 * 256, cu=0) == C["ROPE_QK_ERR_NULL"]  # head-major [H, T, D] view


def test_positions_entry_errors():
    assert lib.rope_qk_positions(ctypes.c_void_p(CU), 4, -1, ctypes.c_void_p(Q), None) == C["ROPE_QK_ERR_SHAPE"]
    assert lib.rope_qk_positions(ctypes.c_void_p(CU), -1, 8, ctypes.c_void_p(Q), None) == C["ROPE_QK_ERR_SHAPE"]
    assert lib.rope_qk_positions(None, 4, 8, ctypes.c_void_p(Q), None) == C["ROPE_QK_ERR_NULL"]
    assert lib.rope_qk_positions(ctypes.c_void_p(CU), 4, 8, None, None) == C["ROPE_QK_ERR_NULL"]
    assert lib.rope_qk_positions(ctypes.c_void_p(CU), 4, 0, None, None) == C["ROPE_QK_OK"]


def test_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        P.rope_qk_fwd(q, k, cu, 1e4)


def test_library_shares_torchs_hip_runtime():
    """The binding loads torch first, so one libamdhip64 instance serves torch and the library."""
    maps = open("/proc/self/maps").read()
    hips = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(hips) == 1, hips


def fwd_opt(opts, which="rope_qk_fwd_opt", **kw):
    args = dict(q=Q, k=K, cu=CU, nseq=4, T=256, Hq=14, Hkv=2, D=64, theta=1e6, dtype=1)
    args.update(kw)
    D, Hq, Hkv = args["D"], args["Hq"], args["Hkv"]
    return getattr(lib, which)(ctypes.c_void_p(args["q"]), ctypes.c_void_p(args["k"]), ctypes.c_void_p(args["cu"]),
                               args["nseq"], args["T"], Hq, Hkv, D, Hq * D, D, Hkv * D, D, args["theta"],
                               args["dtype"], ctypes.byref(opts) if opts is not None else None, None)


LLAMA3 = dict(factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0, original_max_position=8192.0)


@pytest.mark.parametrize("which", ["rope_qk_fwd_opt", "rope_qk_bwd_opt"])
def test_option_error_codes(which):
    E = C["ROPE_QK_ERR_OPTION"]
    f = lambda o, **kw: fwd_opt(o, which=which, **kw)  # noqa: E731
    mk = P.make_options
    assert f(mk(pos_offset=-1)) == E
    assert f(mk(pos_offset=2 ** 31 - 256)) == E  # pos_offset + T past 2^31 - 1
    assert f(mk(pos_offset=2 ** 31 - 257), cu=0) == C["ROPE_QK_ERR_NULL"]  # just fits: reaches the next check
    for r in (1, 3, 66, 128):  # odd, odd, > D, > D
        assert f(mk(rotary_dim=r)) == E, r
    o = mk()
    o.pairing = 5
    assert f(o) == E
    o = mk()
    o.scaling = 7
    assert f(o) == E
    o = mk()
    o.freq_precision = 2
    assert f(o) == E
    o = mk()
    o.reserved = 1
    assert f(o) == E
    assert f(mk(freq_fp32=True), cu=0) == C["ROPE_QK_ERR_NULL"]
    for bad in (dict(factor=0.0), dict(high_freq_factor=1.0), dict(original_max_position=0.0),
                dict(low_freq_factor=0.0), dict(factor=float("inf"))):
        assert f(mk(llama3={**LLAMA3, **bad})) == E, bad
    # options are checked before the no-op shapes return
    assert f(mk(rotary_dim=3), T=0) == E
    # alignment of the rotated part: rotate_half needs (r/2)*elem, interleaved r*elem to be 16-byte multiples
    assert f(mk(rotary_dim=24)) == C["ROPE_QK_ERR_ALIGN"]  # 12 bf16 = 24 bytes
    assert f(mk(rotary_dim=24, interleaved=True), cu=0) == C["ROPE_QK_ERR_NULL"]  # 24 bf16 = 48 bytes: fine
    assert f(mk(rotary_dim=4, interleaved=True)) == C["ROPE_QK_ERR_ALIGN"]  # 8 bytes
    # valid options reach the pointer checks; NULL options behave like the plain call
    assert f(mk(pos_offset=5, rotary_dim=32, interleaved=True, llama3=LLAMA3), cu=0) == C["ROPE_QK_ERR_NULL"]
    assert f(None, dtype=7) == C["ROPE_QK_ERR_DTYPE"]
    assert f(None, T=0) == C["ROPE_QK_OK"]


def test_options_struct_layout_matches_header(tmp_path):
    """The ctypes mirror has the C struct's size and field offsets (gcc on the header)."""
    src = tmp_path / "layout.c"
    names = [n for n, _ in P.RopeQKOptions._fields_]
    body = "".join(f'  printf("%zu\\n", offsetof(rope_qk_options, {n}));\n' for n in names)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "rope_qk.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(rope_qk_options));\n' + body + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(P.RopeQKOptions)] + [getattr(P.RopeQKOptions, n).offset for n in names]
    assert got == want


def test_pairing_and_scaling_constants_match_binding():
    assert C["ROPE_QK_PAIR_HALF"] == P.ROPE_QK_PAIR_HALF and C["ROPE_QK_PAIR_INTERLEAVED"] == P.ROPE_QK_PAIR_INTERLEAVED
    assert C["ROPE_QK_SCALING_NONE"] == P.ROPE_QK_SCALING_NONE
    assert C["ROPE_QK_SCALING_LLAMA3"] == P.ROPE_QK_SCALING_LLAMA3
    assert C["ROPE_QK_FREQ_FP64"] == P.ROPE_QK_FREQ_FP64 and C["ROPE_QK_FREQ_FP32"] == P.ROPE_QK_FREQ_FP32


# ---------------------------------------------------------------------------
# per-head RMSNorm + rotation: argument checks (nothing is launched)
# ---------------------------------------------------------------------------

W_Q, W_K, WS = 4 << 40, 5 << 40, 6 << 40
DWQ, DWK = 7 << 40, 8 << 40


def norm_fwd(q=Q, k=K, qo=None, ko=None, wq=W_Q, wk=W_K, eps=1e-6, cu=CU, nseq=4, T=256, Hq=14, Hkv=2, D=64,
             strides="default", theta=1e6, dtype=1, opts=None):
    qo = q if qo is None else qo
    ko = k if ko is None else ko
    st = None if strides is None else (ctypes.c_int64 * 8)(*(
        [Hq * D, D, Hkv * D, D, Hq * D, D, Hkv * D, D] if strides == "default" else strides))
    return lib.rope_qk_norm_fwd(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(qo), ctypes.c_void_p(ko),
                                ctypes.c_void_p(wq), ctypes.c_void_p(wk), eps, ctypes.c_void_p(cu), nseq, T, Hq, Hkv,
                                D, st, theta, dtype, ctypes.byref(opts) if opts is not None else None, None)


def norm_bwd(ws=WS, ws_size=1 << 30, dwq=DWQ, dwk=DWK, wq=W_Q, eps=1e-6, T=256, Hq=14, Hkv=2, D=64,
             dtype=1, cu=CU, opts=None):
    st = (ctypes.c_int64 * 12)(*([Hq * D, D, Hkv * D, D] * 3))
    return lib.rope_qk_norm_bwd(ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(Q + (1 << 24)),
                                ctypes.c_void_p(K + (1 << 24)), ctypes.c_void_p(Q), ctypes.c_void_p(K),
                                ctypes.c_void_p(wq), ctypes.c_void_p(W_K), eps, ctypes.c_void_p(dwq),
                                ctypes.c_void_p(dwk), ctypes.c_void_p(ws), ws_size, ctypes.c_void_p(cu), 4, T, Hq,
                                Hkv, D, st, 1e6, dtype, ctypes.byref(opts) if opts is not None else None, None)


def test_norm_fwd_error_codes():
    assert norm_fwd(dtype=7) == C["ROPE_QK_ERR_DTYPE"]
    assert norm_fwd(D=96) == C["ROPE_QK_ERR_SHAPE"]  # 12 chunks per head: not a power of two
    assert norm_fwd(D=8) == C["ROPE_QK_ERR_SHAPE"]  # one chunk per head
    assert norm_fwd(D=24, dtype=0) == C["ROPE_QK_ERR_SHAPE"]  # 6 chunks
    assert norm_fwd(Hq=65536, Hkv=1, strides=[65536 * 64, 64, 64, 64, 65536 * 64, 64, 64, 64]) == \
        C["ROPE_QK_ERR_SHAPE"]  # more heads in one tensor than the row division allows
    for eps in (0.0, -1e-6, float("inf"), float("nan")):
        assert norm_fwd(eps=eps) == C["ROPE_QK_ERR_OPTION"], eps
    assert norm_fwd(opts=P.make_options(rotary_dim=32)) == C["ROPE_QK_ERR_OPTION"]  # the norm covers the whole head
    assert norm_fwd(opts=P.make_options(rotary_dim=64), cu=0) == C["ROPE_QK_ERR_NULL"]  # r = D is fine
    assert norm_fwd(strides=None) == C["ROPE_QK_ERR_NULL"]
    assert norm_fwd(wq=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_fwd(wk=0, Hkv=0, strides=[14 * 64, 64, 0, 64, 14 * 64, 64, 0, 64], cu=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_fwd(wq=W_Q + 4) == C["ROPE_QK_ERR_ALIGN"]
    assert norm_fwd(qo=Q + 8 + (1 << 24)) == C["ROPE_QK_ERR_ALIGN"]
    assert norm_fwd(strides=[14 * 64, 32, 2 * 64, 64, 14 * 64, 64, 2 * 64, 64]) == C["ROPE_QK_ERR_LAYOUT"]
    assert norm_fwd(cu=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_fwd(T=0) == C["ROPE_QK_OK"]
    assert norm_fwd(nseq=0) == C["ROPE_QK_OK"]  # in place with nothing inside: no launch
    assert norm_fwd(theta=0.0) == C["ROPE_QK_ERR_THETA"]


def test_norm_bwd_error_codes_and_workspace_size():
    need = lib.rope_qk_norm_bwd_workspace_bytes(256, 14, 2, 64, 1)
    assert need > 0 and need % 16 == 0
    assert lib.rope_qk_norm_bwd_workspace_bytes(256, 14, 2, 64, 9) == C["ROPE_QK_ERR_DTYPE"]
    assert lib.rope_qk_norm_bwd_workspace_bytes(256, 14, 2, 96, 1) == C["ROPE_QK_ERR_SHAPE"]
    assert lib.rope_qk_norm_bwd_workspace_bytes(0, 14, 2, 64, 1) == 0
    # Qwen3-8B-shaped batch: 16 bytes per column for each workgroup, 3072 for
    # 16-bit storage (4 x 3 per compute unit), 4096 for float32 (4 x 4)
    big = lib.rope_qk_norm_bwd_workspace_bytes(65536, 32, 8, 128, 1)
    assert big == 3072 * 2 * 128 * 8
    assert lib.rope_qk_norm_bwd_workspace_bytes(65536, 32, 8, 128, 0) == 4096 * 2 * 128 * 8
    # the largest, as the header states: D = 512 in bf16, 24 MiB (float32
    # rows stop at D = 256: 16 MiB)
    assert lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 512, 1) == 24 << 20
    assert lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 256, 0) == 16 << 20
    assert lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 512, 0) == C["ROPE_QK_ERR_SHAPE"]
    assert norm_bwd(ws=0) == C["ROPE_QK_ERR_WORKSPACE"]
    assert norm_bwd(ws_size=need - 16) == C["ROPE_QK_ERR_WORKSPACE"]
    assert norm_bwd(ws=WS + 8) == C["ROPE_QK_ERR_ALIGN"]
    assert norm_bwd(dwq=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd(dwq=DWQ + 4) == C["ROPE_QK_ERR_ALIGN"]
    assert norm_bwd(eps=0.0) == C["ROPE_QK_ERR_OPTION"]
    assert norm_bwd(wq=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd(cu=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd(dtype=5) == C["ROPE_QK_ERR_DTYPE"]


def norm_bwd_noalloc(dwq=DWQ, dwk=DWK, wq=W_Q, eps=1e-6, T=256, Hq=14, Hkv=2, D=64, dtype=1, cu=CU,
                     opts=None, theta=1e6, strides="default"):
    st = None if strides is None else (ctypes.c_int64 * 12)(*([Hq * D, D, Hkv * D, D] * 3))
    return lib.rope_qk_norm_bwd_noalloc(ctypes.c_void_p(Q), ctypes.c_void_p(K), ctypes.c_void_p(Q + (1 << 24)),
                                        ctypes.c_void_p(K + (1 << 24)), ctypes.c_void_p(Q), ctypes.c_void_p(K),
                                        ctypes.c_void_p(wq), ctypes.c_void_p(W_K), eps, ctypes.c_void_p(dwq),
                                        ctypes.c_void_p(dwk), ctypes.c_void_p(cu), 4, T, Hq, Hkv, D, st, theta, dtype,
                                        ctypes.byref(opts) if opts is not None else None, None)


def test_norm_bwd_noalloc_checks_before_any_hip_call():
    """The no-allocation backward runs every host check of the workspace form,
    in the same order, before it looks up its scratch (the first HIP call)."""
    assert norm_bwd_noalloc(dtype=5) == C["ROPE_QK_ERR_DTYPE"]
    assert norm_bwd_noalloc(D=96) == C["ROPE_QK_ERR_SHAPE"]
    assert norm_bwd_noalloc(D=1024) == C["ROPE_QK_ERR_SHAPE"]
    assert norm_bwd_noalloc(theta=float("nan")) == C["ROPE_QK_ERR_THETA"]
    assert norm_bwd_noalloc(eps=0.0) == C["ROPE_QK_ERR_OPTION"]
    assert norm_bwd_noalloc(opts=P.make_options(rotary_dim=32)) == C["ROPE_QK_ERR_OPTION"]
    assert norm_bwd_noalloc(strides=None) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd_noalloc(wq=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd_noalloc(dwq=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_bwd_noalloc(dwq=DWQ + 4) == C["ROPE_QK_ERR_ALIGN"]
    assert norm_bwd_noalloc(cu=0) == C["ROPE_QK_ERR_NULL"]
    # the same calls give the same codes in the workspace form
    assert norm_bwd(dtype=5) == C["ROPE_QK_ERR_DTYPE"] and norm_bwd(D=96) == C["ROPE_QK_ERR_SHAPE"]
    assert norm_bwd(eps=0.0) == C["ROPE_QK_ERR_OPTION"] and norm_bwd(cu=0) == C["ROPE_QK_ERR_NULL"]
    # every shape the workspace form accepts fits the 24 MiB static scratch
    assert max(lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 512, 1),
               lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 512, 2),
               lib.rope_qk_norm_bwd_workspace_bytes(10 ** 6, 8, 8, 256, 0)) == 24 << 20
    assert "24 MiB" in P.rope_qk_strerror(C["ROPE_QK_ERR_SCRATCH"])


# ---------------------------------------------------------------------------
# tensors that share memory (checked from the pointers and strides)
# ---------------------------------------------------------------------------

def test_q_and_k_that_share_memory_are_refused():
    """q and k are rotated by one launch, so they must share no byte.  D = 72
    (bf16: 72-byte half rows) makes every layout the check accepts stop at
    the alignment check that follows it, so nothing is launched."""
    E, A = C["ROPE_QK_ERR_LAYOUT"], C["ROPE_QK_ERR_ALIGN"]
    T, Hq, Hkv, D, e = 256, 14, 2, 72, 2
    g = lambda **kw: fwd(T=T, Hq=Hq, Hkv=Hkv, D=D, **kw)  # noqa: E731
    assert g() == A  # separate buffers
    assert g(k=Q, kst=Hq * D, ksh=D) == E  # the same tensor passed twice
    assert g(k=Q + Hq * D * e, kst=Hq * D, ksh=D) == E  # k starts at q's second token
    assert g(k=Q + 5 * D * e) == E  # k inside q's rows
    # fused QKV buffer [T, Hq + 2 Hkv, D]: q, k (and v) views with one token stride
    H = Hq + 2 * Hkv
    assert g(qst=H * D, kst=H * D, k=Q + Hq * D * e) == A
    assert g(qst=H * D, kst=H * D, k=Q + (Hq - 1) * D * e) == E  # k's first head is q's last
    assert g(qst=H * D, kst=H * D, k=Q + (Hq + Hkv) * D * e) == A  # k where v would be
    # interleaved heads: q's rows every other head slot, k's in between
    assert g(qst=2 * H * D, qsh=2 * D, kst=2 * H * D, ksh=2 * D, k=Q + D * e) == E  # refused: spans meet
    # head-major views [H, T, D] of one buffer: q heads first, then k heads
    assert g(qst=D, qsh=T * D, kst=D, ksh=T * D, k=Q + Hq * T * D * e) == A
    assert g(qst=D, qsh=T * D, kst=D, ksh=T * D, k=Q + (Hq - 1) * T * D * e) == E


def test_norm_outputs_that_share_memory_are_refused():
    E = C["ROPE_QK_ERR_LAYOUT"]
    # an output over the other tensor's input
    assert norm_fwd(qo=K, cu=0) == E
    # an output partly over its own input (neither in place nor separate)
    assert norm_fwd(qo=Q + 64 * 2, cu=0) == E
    # k_out over q_out
    assert norm_fwd(qo=Q + (1 << 24), ko=Q + (1 << 24) + 64 * 2, cu=0) == E
    # in place and separate outputs pass the check (and stop at the NULL cu_seqlens)
    assert norm_fwd(cu=0) == C["ROPE_QK_ERR_NULL"]
    assert norm_fwd(qo=Q + (1 << 24), ko=K + (1 << 24), cu=0) == C["ROPE_QK_ERR_NULL"]


LAYOUT_DRIVER = r"""
#include <stdio.h>
#include <stdint.h>
#include "rope_layout.h"
int main(void) {
  long long a, Ha, ast, ash, b, Hb, bst, bsh, T, row;
  while (scanf("%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld", &a, &Ha, &ast, &ash, &b, &Hb, &bst, &bsh, &T,
               &row) == 10)
    printf("%d\n", rows_disjoint((const void*)(uintptr_t)a, Ha, ast, ash, (const void*)(uintptr_t)b, Hb, bst, bsh,
                                 T, row) ? 1 : 0);
  return 0;
}
"""


def test_rows_disjoint_never_accepts_an_overlap(tmp_path):
    """The host check against brute force on small byte grids: it never calls
    two grids that share a byte disjoint, and it accepts the fused-projection
    and separate-buffer layouts."""
    import numpy as np

    src = tmp_path / "drv.cpp"
    src.write_text(LAYOUT_DRIVER)
    exe = tmp_path / "drv"
    hdr = os.path.join(ROOT, "packed_varlen_rotary_amd", "csrc")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", hdr, str(src), "-o", str(exe)], check=True)
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(3000):
        T, Ha, Hb = (int(x) for x in rng.integers(1, 5, 3))
        row = int(rng.choice([2, 4, 8]))
        S = int(rng.integers(row, 6 * row))
        ast = S if rng.random() < 0.7 else int(rng.integers(0, 6 * row))
        bst = S if rng.random() < 0.7 else int(rng.integers(0, 6 * row))
        ash, bsh = (int(rng.integers(row, 3 * row)) for _ in range(2))
        a = 1 << 20
        b = a + int(rng.integers(-4 * S, 8 * S))
        cases.append((a, Ha, ast, ash, b, Hb, bst, bsh, T, row))
    # layouts that must be accepted
    cases += [(1 << 20, 4, 96 * 8, 96, (1 << 20) + 4 * 96, 2, 96 * 8, 96, 5, 96),  # fused projection
              (1 << 20, 4, 96, 96 * 7, (1 << 20) + 4 * 96 * 7, 2, 96, 96 * 7, 7, 96)]  # head-major
    inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
    got = [int(x) for x in subprocess.run([str(exe)], input=inp, capture_output=True, text=True,
                                          check=True).stdout.split()]
    for c, g in zip(cases, got):
        a, Ha, ast, ash, b, Hb, bst, bsh, T, row = c
        ba = {a + t * ast + h * ash + i for t in range(T) for h in range(Ha) for i in range(row)}
        bb = {b + t * bst + h * bsh + i for t in range(T) for h in range(Hb) for i in range(row)}
        if g == 1:
            assert not (ba & bb), c
    assert got[-2:] == [1, 1]
    assert sum(got) > 500  # the check is not vacuous
