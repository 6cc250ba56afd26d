"""rope_qk_norm_bwd_noalloc through the C ABI against rope_qk_norm_bwd (needs an MI355X).

The no-allocation form runs the same kernels with the weight-gradient sums in
the library's static per-GPU scratch instead of a caller's workspace, so its
outputs must equal the workspace form's bit for bit (and the workspace form
is checked against the oracle in the norm tests).  Two calls in a row on one
GPU, the second with a smaller input, show that nothing of the first call's
sums leaks into the second.
"""

import numpy as np
import pytest
import torch

import packed_varlen_rotary_amd as P
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-6


def weights(D, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (1.0 + 0.25 * torch.randn(D, generator=g)).float().to(DEV)


def batch(T, Hq, Hkv, D, dtype, cu, seed):
    return {
        "q": W.randn((T, Hq, D), dtype, seed + 1, DEV),
        "k": W.randn((T, Hkv, D), dtype, seed + 2, DEV),
        "dq": W.randn((T, Hq, D), dtype, seed + 3, DEV),
        "dk": W.randn((T, Hkv, D), dtype, seed + 4, DEV),
        "wq": weights(D, seed + 5),
        "wk": weights(D, seed + 6),
        "cu": torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV),
    }


def both_forms(b, theta, in_place=False, stream=None, **opts):
    """(workspace form, no-allocation form) results of one backward."""
    outs = []
    for form in ("workspace", "noalloc"):
        dq_out, dk_out = b["dq"].clone(), b["dk"].clone()
        dq = dq_out if in_place else torch.full_like(dq_out, float("nan"))
        dk = dk_out if in_place else torch.full_like(dk_out, float("nan"))
        dwq = torch.full((b["q"].shape[2],), float("nan"), dtype=torch.float32, device=DEV)
        dwk = torch.full_like(dwq, float("nan"))
        if form == "workspace":
            P.rope_qk_norm_bwd(dq_out, dk_out, b["q"], b["k"], b["wq"], b["wk"], EPS, b["cu"], theta, dq, dk, dwq,
                               dwk, stream=stream, **opts)
        else:
            P.rope_qk_norm_bwd_noalloc(dq_out, dk_out, b["q"], b["k"], b["wq"], b["wk"], EPS, b["cu"], theta, dq, dk,
                                       dwq, dwk, stream=stream, **opts)
        outs.append((dq, dk, dwq, dwk))
    torch.cuda.synchronize()
    return outs


def assert_same(a, b, what):
    for name, x, y in zip(("dq", "dk", "dq_weight", "dk_weight"), a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.uint8) if y.dtype != torch.float32 else y.view(torch.int32)), f"{what}: {name}"


def test_noalloc_matches_workspace_form_two_calls_shrinking():
    # first call: the Qwen3-8B head shape at 8,192 tokens (every backward
    # workgroup busy, the most sums); second: a small batch with far fewer
    # workgroups, whose sums must not pick up the first call's
    rng = np.random.default_rng(11)
    cu1 = np.concatenate([[0], np.sort(rng.integers(1, 8192, size=40)), [8192]])
    big = batch(8192, 32, 8, 128, "bf16", cu1, 100)
    a, b = both_forms(big, 1e6)
    assert_same(a, b, "first call (T=8192)")
    small = batch(300, 6, 2, 128, "bf16", [0, 120, 120, 290], 200)  # empty segment, tail outside
    a, b = both_forms(small, 1e6)
    assert_same(a, b, "second call (T=300)")
    assert torch.isfinite(b[2]).all() and torch.isfinite(b[3]).all()


@pytest.mark.parametrize("T,Hq,Hkv,D,dtype", [
    (65, 3, 2, 512, "bf16"),   # the largest scratch any shape needs: 2 D float64 sums per workgroup at D = 512
    (300, 6, 2, 64, "fp32"),
    (257, 5, 3, 64, "fp16"),
])
def test_noalloc_shapes_in_place_and_options(T, Hq, Hkv, D, dtype):
    b = batch(T, Hq, Hkv, D, dtype, [0, 1, T // 2, T - 3], 300 + D)
    a, c = both_forms(b, 1e6, in_place=True)
    assert_same(a, c, f"in place {dtype} D={D}")
    a, c = both_forms(b, 5e5, pos_offset=77, interleaved=True)
    assert_same(a, c, f"options {dtype} D={D}")


def test_noalloc_on_a_side_stream():
    b = batch(1000, 14, 2, 64, "bf16", [0, 7, 40, 104, 1000], 400)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a, c = both_forms(b, 1e6, stream=side)
    torch.cuda.synchronize()
    assert_same(a, c, "side stream")
