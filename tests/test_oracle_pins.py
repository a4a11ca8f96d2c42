"""Pins of the fp64 oracle against facts it does not compute itself.

Each check compares the oracle with something independent of its own code:
the layer map the pages print, closed forms, library routines the pages name
(F.rms_norm) or that reduce to the definition (scaled_dot_product_attention
with an explicit mask, torch.autograd), central finite differences and
brute-force loops on tiny inputs. The planted-mistake tests at the end show
that plausible bugs in the oracle (a wrong head map, an off-by-one window, a
dropped eps, a dropped term of the norm backward, a misplaced scale) fail at
least one of these pins.
"""

import math
import os

import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as OA

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64) * scale


def _lib_mask(T, W):
    """Band built from library triangle ops (independent of the oracle's predicate)."""
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    if W < 0:
        return causal
    return causal & torch.ones(T, T, dtype=torch.bool).triu(-W)


def _lib_forward(q, k, v, W, scale, qk_norm=True, eps=1e-6):
    """Independent fp64 forward: F.rms_norm + SDPA with an explicit boolean mask + GQA."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if qk_norm:
        q = F.rms_norm(q, (D,), eps=eps)
        k = F.rms_norm(k, (D,), eps=eps)
    qt, kt, vt = (x.permute(0, 2, 1, 3) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=_lib_mask(T, W), scale=scale,
                                       enable_gqa=(Hq != Hkv))
    # LSE from the definition with library routines
    G = Hq // Hkv
    kr = kt.repeat_interleave(G, dim=1)
    S = scale * torch.matmul(qt, kr.transpose(-1, -2))
    S = S.masked_fill(~_lib_mask(T, W), -math.inf)
    lse = torch.logsumexp(S, dim=-1)
    return o.permute(0, 2, 1, 3), lse


# ------------------------------------------------------------------ schedule

def test_sssl_8_layer_map_matches_pages():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "sssl_8layer_map.txt"))
            if ln.strip() and not ln.startswith("#")]
    kinds = [kind for _, kind in rows]
    assert [int(i) for i, _ in rows] == list(range(8))
    for T in (2048, 8192, 101):
        w = oracle.sssl_windows(8, T, "SSSL")
        assert ["global" if x == -1 else "local" for x in w] == kinds
        # local window = half the sequence length
        assert all(x == T // 2 for x in w if x != -1)


def test_sssl_last_layer_forced_global():
    # last layer overridden to L whatever the pattern ([guide] 3.4)
    assert oracle.sssl_windows(6, 2048) == [1024, 1024, 1024, -1, 1024, -1]
    assert oracle.sssl_windows(1, 64, "S") == [-1]
    assert oracle.sssl_windows(3, 64, "SSSS") == [32, 32, -1]
    assert oracle.sssl_windows(4, 64, "L") == [-1, -1, -1, -1]
    with pytest.raises(ValueError):
        oracle.sssl_windows(4, 64, "SXL")


# ------------------------------------------------------------------ band

def _pairs_closed_form(T, W):
    """Number of visible (i, j) pairs: rows i >= W see W+1 keys, rows i < W see i+1."""
    if W < 0 or W >= T - 1:
        return T * (T + 1) // 2
    return (W + 1) * (T - W) + W * (W + 1) // 2


def test_band_mask_against_triangles_and_counts():
    for T in range(1, 41):
        for W in [-1] + list(range(0, T + 3)):
            m = oracle.band_mask(T, W)
            assert torch.equal(m, _lib_mask(T, W)), (T, W)
            assert int(m.sum()) == _pairs_closed_form(T, W), (T, W)


def test_band_mask_special_windows():
    T = 17
    assert torch.equal(oracle.band_mask(T, 0), torch.eye(T, dtype=torch.bool))
    full = oracle.band_mask(T, -1)
    for W in (T - 1, T, 5 * T):
        assert torch.equal(oracle.band_mask(T, W), full)
    # local layers at the pages' shape keep ~75 % of the causal pairs
    assert _pairs_closed_form(2048, 1024) == 1574400
    assert _pairs_closed_form(2048, -1) == 2098176


# ------------------------------------------------------------------ norm

@pytest.mark.parametrize("eps", [1e-6, 0.1, 0.0])
def test_rms_norm_matches_F_rms_norm(eps):
    x = _rand((3, 5, 4, 16), 1)
    x[0, 0, 0] = 0.0  # zero row
    if eps == 0.0:
        x[0, 0, 0] = 1.0
    y, r = oracle.rms_norm(x, eps)
    ref = F.rms_norm(x, (16,), eps=eps)
    assert torch.allclose(y, ref, rtol=1e-14, atol=1e-14)
    # closed form: mean(y^2) = ms / (ms + eps)
    ms = (x * x).mean(-1)
    assert torch.allclose((y * y).mean(-1), ms / (ms + eps), rtol=1e-13, atol=1e-15)


def test_rms_norm_backward_matches_autograd():
    for eps in (1e-6, 0.3):
        x = _rand((4, 7, 2, 8), 2).requires_grad_(True)
        dy = _rand((4, 7, 2, 8), 3)
        y = F.rms_norm(x, (8,), eps=eps)
        (gx,) = torch.autograd.grad(y, x, dy)
        x_hat, r = oracle.rms_norm(x.detach(), eps)
        assert torch.allclose(oracle.rms_norm_backward(x_hat, r, dy), gx, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ forward

FWD_CASES = [
    # B, T, Hq, Hkv, D, W, scale, qk_norm
    (2, 37, 6, 3, 16, -1, None, True),
    (2, 37, 6, 3, 16, 0, None, True),
    (2, 37, 6, 3, 16, 1, None, True),
    (1, 37, 4, 2, 16, 11, 0.7, True),
    (1, 37, 4, 4, 16, 36, None, True),
    (1, 37, 4, 1, 16, 100, None, True),
    (2, 23, 6, 3, 8, 5, 0.5, False),
    (1, 1, 2, 1, 8, -1, None, True),
]


def _fwd_err(case, seed=0):
    B, T, Hq, Hkv, D, W, scale, qk_norm = case
    scale = D ** -0.5 if scale is None else scale
    q, k, v = _rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1), _rand((B, T, Hkv, D), seed + 2)
    o, lse = oracle.attn_forward(q, k, v, W, scale, qk_norm=qk_norm)
    o_ref, lse_ref = _lib_forward(q, k, v, W, scale, qk_norm=qk_norm)
    return max(float((o - o_ref).abs().max()), float((lse - lse_ref).abs().max()))


@pytest.mark.parametrize("case", FWD_CASES)
def test_forward_matches_sdpa_with_explicit_mask(case):
    assert _fwd_err(case) < 1e-12


def test_forward_brute_force_tiny():
    """Pure-Python loops on a tiny case: B=1, T=5, Hq=2, Hkv=1, D=3, W=2."""
    T, D, W, scale, eps = 5, 3, 2, 0.9, 1e-6
    q, k, v = _rand((1, T, 2, D), 11), _rand((1, T, 1, D), 12), _rand((1, T, 1, D), 13)
    o, lse = oracle.attn_forward(q, k, v, W, scale, eps=eps)

    def norm(row):
        r = 1.0 / math.sqrt(sum(float(x) ** 2 for x in row) / len(row) + eps)
        return [float(x) * r for x in row]

    for h in range(2):
        for i in range(T):
            qi = norm(q[0, i, h])
            logits = {}
            for j in range(T):
                if j <= i and i - j <= W:
                    kj = norm(k[0, j, 0])
                    logits[j] = scale * sum(a * b for a, b in zip(qi, kj))
            z = sum(math.exp(s) for s in logits.values())
            assert abs(float(lse[0, h, i]) - math.log(z)) < 1e-12
            for d in range(D):
                ref = sum(math.exp(s) / z * float(v[0, j, 0, d]) for j, s in logits.items())
                assert abs(float(o[0, i, h, d]) - ref) < 1e-12


def test_softmax_rows_sum_to_one_and_vanish_outside_band():
    q, k = _rand((2, 29, 4, 8), 5), _rand((2, 29, 2, 8), 6)
    for W in (-1, 0, 3, 28):
        P = oracle.attention_probs(q, k, W, 0.35)
        assert torch.allclose(P.sum(-1), torch.ones(2, 4, 29, dtype=F64), atol=1e-14)
        assert bool((P[..., ~_lib_mask(29, W)] == 0).all())
        assert bool((P[..., _lib_mask(29, W)] > 0).all())


def test_window_at_least_T_minus_1_is_full_causal_bitwise():
    q, k, v = _rand((1, 19, 4, 8), 7), _rand((1, 19, 2, 8), 8), _rand((1, 19, 2, 8), 9)
    o_full, lse_full = oracle.attn_forward(q, k, v, -1, 0.3)
    for W in (18, 19, 1000):
        o, lse = oracle.attn_forward(q, k, v, W, 0.3)
        assert torch.equal(o, o_full) and torch.equal(lse, lse_full)


def test_window_zero_returns_v_and_self_logit():
    q, k, v = _rand((2, 13, 6, 8), 10), _rand((2, 13, 3, 8), 11), _rand((2, 13, 3, 8), 12)
    o, lse = oracle.attn_forward(q, k, v, 0, 0.4)
    qn, kn = F.rms_norm(q, (8,), eps=1e-6), F.rms_norm(k, (8,), eps=1e-6)
    for h in range(6):
        assert torch.equal(o[:, :, h], v[:, :, h // 2])
        s_ii = 0.4 * (qn[:, :, h] * kn[:, :, h // 2]).sum(-1)
        assert torch.allclose(lse[:, h], s_ii, atol=1e-14)


def test_orthogonal_qk_gives_uniform_softmax():
    """q rows along e0 and k rows along e1 give zero logits: LSE_i = ln(n_i), O_i = band mean of v."""
    T, D = 21, 8
    q = torch.zeros(1, T, 2, D, dtype=F64)
    k = torch.zeros(1, T, 1, D, dtype=F64)
    q[..., 0] = _rand((1, T, 2), 1).abs() + 0.5
    k[..., 1] = _rand((1, T, 1), 2).abs() + 0.5
    v = _rand((1, T, 1, D), 3)
    for W in (-1, 0, 4):
        o, lse = oracle.attn_forward(q, k, v, W, 0.9)
        mask = _lib_mask(T, W).to(F64)
        n = mask.sum(-1)
        assert torch.allclose(lse[0, 0], torch.log(n), atol=1e-14)
        assert torch.allclose(o[0, :, 1], (mask @ v[0, :, 0]) / n[:, None], atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    B, T, Hq, Hkv, D = 2, 15, 6, 2, 8
    q, k, v, do = (_rand((B, T, Hq, D), 20), _rand((B, T, Hkv, D), 21), _rand((B, T, Hkv, D), 22),
                   _rand((B, T, Hq, D), 23))
    G = Hq // Hkv
    kr, vr = k.repeat_interleave(G, dim=2), v.repeat_interleave(G, dim=2)
    for W in (-1, 3):
        o, lse = oracle.attn_forward(q, k, v, W, 0.3)
        o_m, lse_m = oracle.attn_forward(q, kr, vr, W, 0.3)
        assert torch.allclose(o, o_m, atol=1e-15) and torch.allclose(lse, lse_m, atol=1e-15)
        dq, dk, dv = oracle.attn_backward(q, k, v, do, W, 0.3)
        dq_m, dk_m, dv_m = oracle.attn_backward(q, kr, vr, do, W, 0.3)
        assert torch.allclose(dq, dq_m, atol=1e-13)
        assert torch.allclose(dk, dk_m.view(B, T, Hkv, G, D).sum(3), atol=1e-13)
        assert torch.allclose(dv, dv_m.view(B, T, Hkv, G, D).sum(3), atol=1e-13)


def test_norm_makes_output_scale_invariant():
    q, k, v = _rand((1, 31, 4, 16), 30), _rand((1, 31, 2, 16), 31), _rand((1, 31, 2, 16), 32)
    o, _ = oracle.attn_forward(q, k, v, 7, 0.25)
    o8, _ = oracle.attn_forward(8 * q, 8 * k, v, 7, 0.25)
    assert torch.allclose(o, o8, atol=1e-5)


def test_single_position_returns_v0():
    q, k, v = _rand((3, 1, 4, 8), 40), _rand((3, 1, 2, 8), 41), _rand((3, 1, 2, 8), 42)
    o, _ = oracle.attn_forward(q, k, v, -1, 0.3)
    assert torch.equal(o, v.repeat_interleave(2, dim=2))


# ------------------------------------------------------------------ backward

BWD_CASES = [
    (2, 19, 6, 3, 16, -1, True),
    (2, 19, 6, 3, 16, 4, True),
    (1, 19, 4, 4, 8, 0, True),
    (1, 19, 4, 2, 8, 18, True),
    (1, 19, 4, 2, 8, 6, False),
]


def _bwd_err(case, seed=50, scale=0.3):
    B, T, Hq, Hkv, D, W, qk_norm = case
    q, k, v, do = (_rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1),
                   _rand((B, T, Hkv, D), seed + 2), _rand((B, T, Hq, D), seed + 3))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o_ref, _ = _lib_forward(qa, ka, va, W, scale, qk_norm=qk_norm)
    gq, gk, gv = torch.autograd.grad(o_ref, (qa, ka, va), do)
    dq, dk, dv = oracle.attn_backward(q, k, v, do, W, scale, qk_norm=qk_norm)
    return max(float((dq - gq).abs().max()), float((dk - gk).abs().max()), float((dv - gv).abs().max()))


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_autograd_of_library_forward(case):
    assert _bwd_err(case) < 1e-11


@pytest.mark.parametrize("W", [-1, 0, 2, 5])
def test_backward_central_finite_differences(W):
    B, T, Hq, Hkv, D, scale, h = 1, 6, 4, 2, 8, 0.35, 1e-6
    q, k, v, do = (_rand((B, T, Hq, D), 60), _rand((B, T, Hkv, D), 61), _rand((B, T, Hkv, D), 62),
                   _rand((B, T, Hq, D), 63))
    grads = oracle.attn_backward(q, k, v, do, W, scale)

    def loss(qq, kk, vv):
        return float((oracle.attn_forward(qq, kk, vv, W, scale)[0] * do).sum())

    for idx, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = torch.zeros_like(x)
        flat, fdf = x.view(-1), fd.view(-1)
        for e in range(flat.numel()):
            old = float(flat[e])
            flat[e] = old + h
            args = [q, k, v]
            lp = loss(*args)
            flat[e] = old - h
            lm = loss(*args)
            flat[e] = old
            fdf[e] = (lp - lm) / (2 * h)
        # W = 0 leaves dq and dk exactly zero, so the bound is relative to max(|g|, 1)
        err = float((fd - g).norm() / max(float(g.norm()), 1.0))
        assert err < 1e-6, (idx, err)


def test_delta_identity():
    """Delta_i = <dO_i, O_i> equals sum_j P_ij <dO_i, v_j>."""
    q, k, v, do = _rand((1, 17, 4, 8), 70), _rand((1, 17, 2, 8), 71), _rand((1, 17, 2, 8), 72), _rand((1, 17, 4, 8), 73)
    o, _ = oracle.attn_forward(q, k, v, 5, 0.3)
    P = oracle.attention_probs(q, k, 5, 0.3)
    vr = v.repeat_interleave(2, dim=2)
    dP = torch.einsum("bihd,bjhd->bhij", do, vr)
    assert torch.allclose(oracle.attn_backward_delta(o, do), (P * dP).sum(-1), atol=1e-13)


# ------------------------------------------------------------------ rotary embedding

def _lib_rope(x, theta):
    """Rotary embedding by complex multiplication (torch.polar): the pair
    (x_i, x_{i+D/2}) as the complex number x_i + 1j x_{i+D/2}, times e^{1j theta[t, i]}."""
    T, D = x.shape[1], x.shape[-1]
    z = torch.complex(x[..., : D // 2].contiguous(), x[..., D // 2:].contiguous())
    w = torch.polar(torch.ones_like(theta[:T]), theta[:T]).view(1, T, 1, D // 2)
    y = z * w
    return torch.cat([y.real, y.imag], dim=-1)


def test_rope_angles_geometric_ladder():
    """theta[t, i] = t * base^(-2i/D): row 1 is torch.logspace from 1 down to
    base^(-(D-2)/D), and every row t is t times row 1."""
    for D, base in ((16, 10000.0), (128, 10000.0), (8, 500.0)):
        th = oracle.rope_angles(7, D, base)
        ladder = torch.logspace(0.0, -(D - 2) / D, D // 2, base=base, dtype=F64)
        assert torch.allclose(th[1], ladder, rtol=1e-14, atol=0)
        assert torch.equal(th[0], torch.zeros(D // 2, dtype=F64))
        assert torch.allclose(th, torch.arange(7, dtype=F64).view(7, 1) * ladder, rtol=1e-14, atol=0)


def test_rope_rotation_is_complex_multiplication():
    x = _rand((2, 9, 3, 16), 80)
    theta = oracle.rope_angles(12, 16)
    cos, sin = oracle.rope_tables(12, 16)
    assert torch.allclose(oracle.rope_rotate(x, cos, sin), _lib_rope(x, theta), atol=1e-14)


def test_rope_preserves_norm_and_inverts():
    x = _rand((1, 11, 2, 32), 81, scale=3.0)
    cos, sin = oracle.rope_tables(11, 32)
    y = oracle.rope_rotate(x, cos, sin)
    assert torch.allclose(y.norm(dim=-1), x.norm(dim=-1), rtol=1e-14)
    assert torch.allclose(oracle.rope_rotate_back(y, cos, sin), x, atol=1e-14)
    assert torch.equal(y[:, 0], x[:, 0])  # position 0 turns by zero


def test_rope_scores_depend_on_offset_only():
    """<R_m q, R_n k> = <R_{m+s} q, R_{n+s} k>: the logit sees only m - n."""
    D, T = 16, 40
    cos, sin = oracle.rope_tables(T, D)
    q1, k1 = _rand((D,), 82), _rand((D,), 83)
    q = torch.zeros(1, T, 1, D, dtype=F64)
    k = torch.zeros(1, T, 1, D, dtype=F64)
    q[0, :, 0] = q1
    k[0, :, 0] = k1
    qr, kr = oracle.rope_rotate(q, cos, sin)[0, :, 0], oracle.rope_rotate(k, cos, sin)[0, :, 0]
    for m, n, sft in ((5, 2, 7), (3, 3, 30), (10, 0, 19), (0, 9, 11)):
        assert abs(float(qr[m] @ kr[n]) - float(qr[m + sft] @ kr[n + sft])) < 1e-12
    assert abs(float(qr[4] @ kr[1]) - float(qr[3] @ kr[1])) > 1e-3  # and it does see the offset


def test_rope_commutes_with_the_weightless_norm():
    x = _rand((2, 13, 3, 16), 84, scale=2.0)
    cos, sin = oracle.rope_tables(13, 16)
    a = oracle.rms_norm(oracle.rope_rotate(x, cos, sin), 1e-6)[0]
    b = oracle.rope_rotate(oracle.rms_norm(x, 1e-6)[0], cos, sin)
    assert torch.allclose(a, b, atol=1e-14)


ROPE_CASES = [
    # B, T, Hq, Hkv, D, W, qk_norm
    (2, 21, 6, 3, 16, -1, True),
    (1, 21, 4, 4, 8, 5, True),
    (1, 21, 4, 2, 16, 0, True),
    (1, 21, 4, 2, 8, 7, False),
]


def _rope_err(case, seed=90, scale=0.4):
    B, T, Hq, Hkv, D, W, qk_norm = case
    q, k, v, do = (_rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1),
                   _rand((B, T, Hkv, D), seed + 2), _rand((B, T, Hq, D), seed + 3))
    theta = oracle.rope_angles(T + 5, D)  # longer table than T: rows 0 .. T-1 are used
    rope = (torch.cos(theta), torch.sin(theta))
    o, lse = oracle.attn_forward(q, k, v, W, scale, qk_norm=qk_norm, rope=rope)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o_ref, lse_ref = _lib_forward(_lib_rope(qa, theta), _lib_rope(ka, theta), va, W, scale, qk_norm=qk_norm)
    gq, gk, gv = torch.autograd.grad(o_ref, (qa, ka, va), do)
    dq, dk, dv = oracle.attn_backward(q, k, v, do, W, scale, qk_norm=qk_norm, rope=rope)
    return max(float((o - o_ref).abs().max()), float((lse - lse_ref).abs().max()),
               float((dq - gq).abs().max()), float((dk - gk).abs().max()), float((dv - gv).abs().max()))


@pytest.mark.parametrize("case", ROPE_CASES)
def test_rope_attention_matches_library_forward_and_autograd(case):
    assert _rope_err(case) < 1e-11


def test_rope_backward_central_finite_differences():
    B, T, Hq, Hkv, D, W, scale, h = 1, 6, 2, 1, 8, 3, 0.35, 1e-6
    q, k, v, do = (_rand((B, T, Hq, D), 95), _rand((B, T, Hkv, D), 96), _rand((B, T, Hkv, D), 97),
                   _rand((B, T, Hq, D), 98))
    rope = oracle.rope_tables(T, D, base=30.0)  # fast-turning table: large angles at small T
    grads = oracle.attn_backward(q, k, v, do, W, scale, rope=rope)

    def loss():
        return float((oracle.attn_forward(q, k, v, W, scale, rope=rope)[0] * do).sum())

    for idx, (x, g) in enumerate(zip((q, k), grads[:2])):
        fd = torch.zeros_like(x)
        flat, fdf = x.view(-1), fd.view(-1)
        for e in range(flat.numel()):
            old = float(flat[e])
            flat[e] = old + h
            lp = loss()
            flat[e] = old - h
            lm = loss()
            flat[e] = old
            fdf[e] = (lp - lm) / (2 * h)
        assert float((fd - g).norm() / g.norm()) < 1e-6, idx


# ------------------------------------------------------------------ value embeddings

def test_ve_layers_match_the_printed_map():
    rows = [int(ln) for ln in open(os.path.join(GOLDEN, "ve_layers_depth8.txt")) if ln.strip() and ln[0] != "#"]
    assert oracle.ve_layers(8) == rows
    for n in (1, 2, 5, 12):
        layers = oracle.ve_layers(n)
        assert layers[-1] == n - 1 and all(b - a == 2 for a, b in zip(layers, layers[1:]))


def test_ve_zero_gate_weights_give_the_identity_pathway():
    """Zero gate weights: 2 sigmoid(0) = 1, so v' = v + ve (the trainer's initial state)."""
    B, T, Hkv, D, V = 2, 5, 3, 8, 11
    v, x32, table = _rand((B, T, Hkv, D), 1), _rand((B, T, 32), 2), _rand((V, Hkv * D), 3)
    ids = torch.randint(0, V, (B, T), generator=torch.Generator().manual_seed(4))
    w = torch.zeros(Hkv, 32, dtype=F64)
    assert torch.equal(oracle.ve_gate(x32, w), torch.ones(B, T, Hkv, dtype=F64))
    assert torch.allclose(oracle.ve_mix(v, x32, w, ids, table), v + table[ids].view(B, T, Hkv, D), atol=0)


VE_CASES = [
    # B, T, Hq, Hkv, D, W, V
    (2, 17, 6, 3, 16, -1, 13),
    (1, 17, 4, 4, 8, 5, 7),
]


def _ve_inputs(case, seed):
    B, T, Hq, Hkv, D, W, V = case
    q, k, v, do = (_rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1),
                   _rand((B, T, Hkv, D), seed + 2), _rand((B, T, Hq, D), seed + 3))
    x32, w, table = _rand((B, T, 32), seed + 4), _rand((Hkv, 32), seed + 5, 0.2), _rand((V, Hkv * D), seed + 6)
    ids = torch.randint(0, V, (B, T), generator=torch.Generator().manual_seed(seed + 7))
    return q, k, v, do, x32, w, ids, table


def _ve_err(case, seed=120, scale=0.4):
    B, T, Hq, Hkv, D, W, V = case
    q, k, v, do, x32, w, ids, table = _ve_inputs(case, seed)
    o, lse = oracle.attn_forward(q, k, v, W, scale, ve=(x32, w, ids, table))
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, x32, w, table)]
    qa, ka, va, xa, wa, ta = leaves
    gate = 2.0 * torch.sigmoid(F.linear(xa, wa))
    vm = va + gate.unsqueeze(-1) * F.embedding(ids, ta).view(B, T, Hkv, D)
    o_ref, lse_ref = _lib_forward(qa, ka, vm, W, scale)
    gq, gk, gv, gx, gw, gt = torch.autograd.grad(o_ref, leaves, do)
    dq, dk, dv, dve, dw, dx32 = oracle.attn_backward(q, k, v, do, W, scale, ve=(x32, w, ids, table))
    # the table's gradient is the per-position dve summed into the rows the ids pick
    dtable = torch.zeros_like(table).index_add_(0, ids.view(-1), dve.reshape(B * T, Hkv * D))
    return max(float((o - o_ref).abs().max()), float((lse - lse_ref).abs().max()),
               float((dq - gq).abs().max()), float((dk - gk).abs().max()), float((dv - gv).abs().max()),
               float((dx32 - gx).abs().max()), float((dw - gw).abs().max()), float((dtable - gt).abs().max()))


@pytest.mark.parametrize("case", VE_CASES)
def test_ve_attention_matches_library_forward_and_autograd(case):
    assert _ve_err(case) < 1e-11


def test_ve_backward_central_finite_differences():
    case = (1, 6, 2, 1, 8, 3, 5)
    q, k, v, do, x32, w, ids, table = _ve_inputs(case, 130)
    h, scale = 1e-6, 0.35
    grads = oracle.attn_backward(q, k, v, do, 3, scale, ve=(x32, w, ids, table))

    def loss():
        return float((oracle.attn_forward(q, k, v, 3, scale, ve=(x32, w, ids, table))[0] * do).sum())

    for x, g in ((w, grads[4]), (x32, grads[5])):
        fd = torch.zeros_like(x)
        flat, fdf = x.view(-1), fd.view(-1)
        for e in range(flat.numel()):
            old = float(flat[e])
            flat[e] = old + h
            lp = loss()
            flat[e] = old - h
            lm = loss()
            flat[e] = old
            fdf[e] = (lp - lm) / (2 * h)
        assert float((fd - g).norm() / g.norm()) < 1e-6


# ------------------------------------------------------------------ planted mistakes

def _all_pins_pass():
    """Run a cheap selection of the pins above; True if all of them hold."""
    if _fwd_err(FWD_CASES[0]) > 1e-12 or _fwd_err(FWD_CASES[3]) > 1e-12 or _fwd_err(FWD_CASES[2]) > 1e-12:
        return False
    if _bwd_err(BWD_CASES[1]) > 1e-11:
        return False
    for T in (9, 16):
        for W in (-1, 0, 3):
            if int(OA.band_mask(T, W).sum()) != _pairs_closed_form(T, W):
                return False
    x = _rand((2, 3, 8), 3)
    if not torch.allclose(OA.rms_norm(x, 0.1)[0], F.rms_norm(x, (8,), eps=0.1), atol=1e-14):
        return False
    if _rope_err(ROPE_CASES[0]) > 1e-11 or _rope_err(ROPE_CASES[1]) > 1e-11:
        return False
    if _ve_err(VE_CASES[0]) > 1e-11:
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _all_pins_pass()


def _mut_kv_head(h, Hq, Hkv):
    return h % Hkv


def _mut_band_mask(T, window):
    i = torch.arange(T).view(T, 1)
    j = torch.arange(T).view(1, T)
    vis = j <= i
    if window >= 0:
        vis = vis & ((i - j) < window)  # off by one: W keys instead of W + 1
    return vis


def _mut_rms_norm(x, eps):
    x = x.to(F64)
    r = 1.0 / torch.sqrt((x * x).mean(dim=-1, keepdim=True))  # eps dropped
    return x * r, r


def _mut_rms_norm_backward(x_hat, r, dx_hat):
    return r * dx_hat  # projection term dropped


def _mut_rope_rotate(x, cos, sin):
    x = x.to(F64)
    T, D = x.shape[1], x.shape[-1]
    c = cos[:T].to(F64).view(1, T, 1, D // 2)
    s = sin[:T].to(F64).view(1, T, 1, D // 2)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return torch.cat([x1 * c + x2 * s, -x1 * s + x2 * c], dim=-1)  # turns the other way


def _mut_rope_rotate_back(y, cos, sin):
    return OA.rope_rotate(y, cos, sin)  # the rotation instead of its transpose


def _mut_ve_gate(x32, w):
    return torch.sigmoid(x32.to(F64) @ w.to(F64).transpose(0, 1))  # factor 2 dropped


def _mut_ve_backward(dv_mixed, x32, w, ids, table):
    B, T, Hkv, D = dv_mixed.shape
    dvm = dv_mixed.to(F64)
    ve = table.to(F64)[ids.long()].view(B, T, Hkv, D)
    g = OA.ve_gate(x32, w)
    dz = (dvm * ve).sum(-1) * g * (1.0 - g)  # slope of sigmoid taken at g instead of g/2
    return g.unsqueeze(-1) * dvm, torch.einsum("bth,btc->hc", dz, x32.to(F64)), dz @ w.to(F64)


def _mut_probs(q_hat_bh, k_hat_bg, mask, scale):
    return OA.__dict__["_real_probs"](q_hat_bh, k_hat_bg, mask, scale * scale)  # scale applied twice


@pytest.mark.parametrize("name,mutant", [
    ("kv_head", _mut_kv_head),
    ("band_mask", _mut_band_mask),
    ("rms_norm", _mut_rms_norm),
    ("rms_norm_backward", _mut_rms_norm_backward),
    ("_probs_one_head", _mut_probs),
    ("rope_rotate", _mut_rope_rotate),
    ("rope_rotate_back", _mut_rope_rotate_back),
    ("ve_gate", _mut_ve_gate),
    ("ve_backward", _mut_ve_backward),
])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setitem(OA.__dict__, "_real_probs", OA._probs_one_head)
    monkeypatch.setattr(OA, name, mutant)
    assert not _all_pins_pass(), f"planted mistake in {name} went unnoticed"


@pytest.mark.parametrize("W,Hq,Hkv", [(-1, 4, 2), (5, 6, 3), (0, 2, 2), (12, 4, 1)])
def test_row_sampled_forward_equals_the_full_forward(W, Hq, Hkv):
    """attn_forward_rows (used to sample every (batch, head) of full-size
    layers) is the full forward restricted to the rows asked for, in any order,
    with or without the norm."""
    B, T, D = 2, 37, 16
    g = torch.Generator().manual_seed(31 + W)
    q = torch.randn(B, T, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, T, Hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, T, Hkv, D, generator=g, dtype=torch.float64)
    rows = [36, 0, 17, 5, 5, 30]
    for qk_norm in (True, False):
        o, lse = oracle.attn_forward(q, k, v, W, 0.3, qk_norm=qk_norm)
        o_r, lse_r = oracle.attn_forward_rows(q, k, v, rows, W, 0.3, qk_norm=qk_norm)
        assert torch.allclose(o_r, o[:, rows], rtol=0, atol=1e-12)
        assert torch.allclose(lse_r, lse[:, :, rows], rtol=0, atol=1e-12)
    # the absolute weighted sum: P |v| with the full forward's probabilities, never below |O|
    _, _, o_abs = oracle.attn_forward_rows(q, k, v, rows, W, 0.3, with_abs=True)
    P = oracle.attention_probs(q, k, W, 0.3)  # [B, Hq, T, T]
    G = Hq // Hkv
    for h in range(Hq):
        want = P[:, h][:, rows] @ v[:, :, h // G].abs()
        assert torch.allclose(o_abs[:, :, h], want, rtol=0, atol=1e-12)
    o, _ = oracle.attn_forward(q, k, v, W, 0.3)
    assert bool((o_abs >= o[:, rows].abs() - 1e-12).all())
