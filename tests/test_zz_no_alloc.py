"""GPU check of the no-allocation backward (sa_attn_bwd_noalloc): on two calls
in a row, the second with a smaller input, its outputs are bit-identical to
sa_attn_bwd's on the same inputs (the same kernels run; only the scratch
differs), so the shared scratch keeps nothing from one call to the next that
the result depends on."""

import pytest
import torch

import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import qk_normed_sliding_amd as pkg
    return pkg


CASES = [  # B, T, Hq, Hkv, D, W, seed: the second call is the smaller one
    (2, 300, 6, 3, 128, 100, 71),
    (1, 130, 4, 2, 64, -1, 72),
]


def test_noalloc_backward_matches_the_workspace_backward(sa):
    outs = []
    for B, T, Hq, Hkv, D, W, seed in CASES:
        log(f"[no-alloc backward] B{B} T{T} Hq{Hq} Hkv{Hkv} D{D} W{W}")
        q, k, v, do = (x.cuda() for x in synth.small_case(B, T, Hq, Hkv, D, seed=seed))
        scale = D ** -0.5
        o, lse = sa.sa_attn_fwd(q, k, v, window=W, softmax_scale=scale)
        ref = sa.sa_attn_bwd(q, k, v, o, lse, do, window=W, softmax_scale=scale)
        got = sa.sa_attn_bwd_noalloc(q, k, v, o, lse, do, window=W, softmax_scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.isfinite(a.float()).all(), name
            assert torch.equal(a, b), f"{name} differs from sa_attn_bwd"
        outs.append(got)
    # the first call's outputs were not touched by the second call
    assert all(torch.isfinite(t.float()).all() for t in outs[0])
