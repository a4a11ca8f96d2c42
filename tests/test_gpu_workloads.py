"""Parity at the full workload sizes, in the launch configuration the benchmark
times (one sa_attn_fwd + sa_attn_bwd call per layer over the whole batch).

The GPU computes every layer at full size; the fp64 oracle recomputes whole
(batch, KV-head group) slices of it — each slice is an independent instance
of the same definition (its query heads, its KV head, all T positions) — and
the slice's outputs and gradients are compared element by element.

Workload 5 scales a seeded 10 % of the head rows of q, k, v and dO by 8. With
v rows scaled, |O| reaches ~15-26, where one bf16 step is 0.0625-0.125, so
storing O in bf16 alone can exceed a 2e-2 absolute bound. For that workload O
is held to |diff| <= 2e-2 + 2^-7 |O_ref| elementwise (one bf16 step relative
on top of the absolute bound), and a variant that scales only q and k (the
rows that reach the softmax) is held to the plain 2e-2 bound. On the rows
sampled across every (batch, head) the relative part is taken of sum_j P_ij
|v_j| rather than of |O_ref|: the bf16 rounding of the probabilities and of
O scales with that sum, which exceeds |O_ref| where large scaled values of
opposite signs nearly cancel in the average.
"""

import pytest
import torch

import synth
from gpu_helpers import compare_backward, compare_forward, gpu_fwd_bwd, log, set_cpu_threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    set_cpu_threads()
    import qk_normed_sliding_amd as pkg
    return pkg


def _check_slices(w, layer, q, k, v, do, out, slices, o_rel=0.0, rope=None, ve=None):
    o, lse, dq, dk, dv = out
    W = w.windows[layer]
    G = w.Hq // w.Hkv
    for b, g in slices:
        hs = slice(g * G, (g + 1) * G)
        ks = slice(g, g + 1)
        ve_slice = None
        if ve is not None:  # the slice's own rows, gate weights and table columns of KV head g
            x, gw, ids, table = ve
            ve_slice = (x[b:b + 1, :, :32], gw[g:g + 1], ids[b:b + 1], table[:, g * w.D:(g + 1) * w.D])
        log(f"  layer {layer} W={W} slice b={b} g={g}")
        qs, kk, vs, ds = q[b:b + 1, :, hs], k[b:b + 1, :, ks], v[b:b + 1, :, ks], do[b:b + 1, :, hs]
        os_, ls = o[b:b + 1, :, hs], lse[b:b + 1, hs]
        if o_rel > 0:
            import oracle
            if ve_slice is None:
                # relative part of sum_j P_ij |v_j| (see the module docstring)
                o_ref, lse_ref, o_scale = oracle.attn_forward_rows(qs, kk, vs, range(w.T), W, w.scale, eps=w.eps,
                                                                   with_abs=True)
            else:
                o_ref, lse_ref = oracle.attn_forward(qs, kk, vs, W, w.scale, eps=w.eps, ve=ve_slice)
                o_scale = o_ref.abs()
            diff = (os_.cpu().double() - o_ref).abs()
            bound = 2e-2 + o_rel * o_scale
            log(f"  O max-abs {float(diff.max()):.3e} (mixed bound), LSE max-abs "
                f"{float((ls.cpu().double() - lse_ref).abs().max()):.3e}")
            assert bool((diff <= bound).all())
            assert float((ls.cpu().double() - lse_ref).abs().max()) <= 2e-2
        else:
            compare_forward(os_, ls, qs, kk, vs, W, w.scale, eps=w.eps, rope=rope)
        compare_backward(dq[b:b + 1, :, hs], dk[b:b + 1, :, ks], dv[b:b + 1, :, ks], qs, kk, vs, ds, W, w.scale,
                         eps=w.eps, rope=rope, ve=ve_slice)


def _check_rows(w, layer, q, k, v, o, lse, o_rel=0.0, n_random=4):
    """Every (batch, head) of the full-size layer, on sampled query rows: the
    first rows (few keys), the middle, the last, and seeded random ones,
    against the oracle's row-by-row forward."""
    import oracle

    T = w.T
    g = torch.Generator().manual_seed(1000 + layer)
    rows = sorted({0, 1, 2, 3, T // 2, T - 1} | set(torch.randint(0, T, (n_random,), generator=g).tolist()))
    o_ref, lse_ref, o_abs = oracle.attn_forward_rows(q, k, v, rows, w.windows[layer], w.scale, eps=w.eps,
                                                     with_abs=True)
    got_o = o.cpu()[:, rows].double()
    diff = (got_o - o_ref).abs()
    bound = 2e-2 + o_rel * o_abs
    el = float((lse.cpu()[:, :, rows].double() - lse_ref).abs().max())
    log(f"  all {w.B}x{w.Hq} (batch, head) on rows {rows}: O max-abs {float(diff.max()):.3e}, LSE max-abs {el:.3e}")
    assert bool((diff <= bound).all())
    assert el <= 2e-2


@pytest.mark.parametrize("cfg", [2, 3])
def test_single_layer_workloads(sa, cfg):
    w = synth.WORKLOADS[cfg]
    log(f"[workload {cfg}] {w.name}")
    q, k, v, do = synth.layer_inputs(w, 0)
    out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[0], w.scale, eps=w.eps)
    _check_slices(w, 0, q, k, v, do, out, [(0, 0), (w.B - 1, w.Hkv - 1)])


def test_sssl_stack_workload(sa):
    w = synth.WORKLOADS[4]
    log(f"[workload 4] {w.name}")
    for layer in range(w.n_layer):
        q, k, v, do = synth.layer_inputs(w, layer)
        out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[layer], w.scale, eps=w.eps)
        _check_slices(w, layer, q, k, v, do, out, [(layer % w.B, layer % w.Hkv)])
        _check_rows(w, layer, q, k, v, out[0], out[1])


@pytest.mark.parametrize("layer", list(range(8)))
def test_long_context_workload(sa, layer):
    """All 8 layers of the long-context stack at full size: one (batch, KV
    group) slice each against the oracle, and every (batch, head) on sampled
    rows."""
    w = synth.WORKLOADS[5]
    log(f"[workload 5] {w.name} layer {layer}")
    q, k, v, do = synth.layer_inputs(w, layer)
    out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[layer], w.scale, eps=w.eps)
    _check_slices(w, layer, q, k, v, do, out, [(layer % w.B, layer % w.Hkv)], o_rel=2.0 ** -7)
    _check_rows(w, layer, q, k, v, out[0], out[1], o_rel=2.0 ** -7)


def test_long_context_qk_rows_only(sa):
    w = synth.WORKLOADS[5]
    log(f"[workload 5, q/k rows scaled only] layer 6")
    q, k, v, do = synth.layer_inputs(w, 6, qk_rows_only=True)
    out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[6], w.scale, eps=w.eps)
    _check_slices(w, 6, q, k, v, do, out, [(2, 2)])


@pytest.mark.parametrize("layer", [0, 3])
def test_mha_model_shape_workload(sa, layer):
    """The pages' own model shape (MHA, n_head = n_kv_head = 6, device batch
    128): one sliding and one full-causal layer at full size, each slice
    (batch row, head) compared with the oracle."""
    w = synth.WORKLOADS[6]
    log(f"[workload 6] {w.name} layer {layer}")
    q, k, v, do = synth.layer_inputs(w, layer)
    out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[layer], w.scale, eps=w.eps)
    _check_slices(w, layer, q, k, v, do, out, [(0, 0), (w.B - 1, w.Hkv - 1), (61 + layer, 2 + layer % 3)])


@pytest.mark.parametrize("layer", [2, 3])
def test_sssl_stack_with_rope(sa, layer):
    """A sliding and a full-causal layer of the 8-layer stack with the rotary
    embedding fused, tables precomputed for ten sequence lengths."""
    w = synth.WORKLOADS[4]
    log(f"[workload 4 + rope] layer {layer}")
    q, k, v, do = synth.layer_inputs(w, layer)
    rope = sa.rope_tables(10 * w.T, w.D, device="cuda")
    out = gpu_fwd_bwd(sa, q, k, v, do, w.windows[layer], w.scale, eps=w.eps, rope=rope)
    _check_slices(w, layer, q, k, v, do, out, [(3 + layer, 1), (w.B - 1, 2)], rope=rope)


@pytest.mark.parametrize("layer", [1, 3])
def test_sssl_stack_with_value_embeddings(sa, layer):
    """Layers 1 (sliding) and 3 (full causal) of the stack carry value
    embeddings in the trainer: full-size call with the gate fused; each
    (batch row, KV group) slice against the oracle on its own gate inputs."""
    import oracle

    w = synth.WORKLOADS[4]
    log(f"[workload 4 + value embeddings] layer {layer}")
    q, k, v, do = synth.layer_inputs(w, layer)
    ve = synth.ve_inputs(w, layer)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    ve_d = tuple(t.cuda() for t in ve)
    W = w.windows[layer]
    o, lse = sa.sa_attn_fwd(qd, kd, vd, window=W, softmax_scale=w.scale, eps=w.eps, ve=ve_d)
    dq, dk, dv, dve, dw, dx32 = sa.sa_attn_bwd(qd, kd, vd, o, lse, dod, window=W, softmax_scale=w.scale, eps=w.eps,
                                               ve=ve_d)
    torch.cuda.synchronize()
    _check_slices(w, layer, q, k, v, do, (o, lse, dq, dk, dv), [(5, 1), (w.B - 2, 2)], o_rel=2.0 ** -7, ve=ve)
    # dw and dx32 sum over every position and head: checked whole against the oracle's gate backward,
    # given the GPU's own dL/dv' (the attention part is checked above)
    x, gw, ids, table = ve
    _, dw_r, dx_r = oracle.ve_backward(dv.cpu(), x[..., :32], gw, ids, table)
    from gpu_helpers import rel_l2
    e_w, e_x = rel_l2(dw.cpu(), dw_r), rel_l2(dx32.cpu(), dx_r)
    log(f"  dw rel-L2 {e_w:.3e}  dx32 rel-L2 {e_x:.3e}")
    assert e_w <= 5e-2 and e_x <= 5e-2


@pytest.mark.parametrize("layer", [1, 3])
def test_value_embedding_gate_gradients_full_size(sa, layer):
    """The gate's weight and input gradients at full size, against the oracle
    alone. dW sums over every position and head, so the full-size call gets an
    upstream gradient that is zero outside batch row b0: dW, dx32 and dve then
    hold that row's contributions only, which the oracle computes from the
    row's q, k, v, dO and gate inputs over all its KV heads (no GPU value
    enters the reference). Rows with zero upstream gradient must give exactly
    zero gradients."""
    import oracle
    from gpu_helpers import rel_l2

    w = synth.WORKLOADS[4]
    b0 = 2 + layer
    log(f"[workload 4 + value embeddings, dO in batch row {b0} only] layer {layer}")
    q, k, v, do = synth.layer_inputs(w, layer)
    do_z = torch.zeros_like(do)
    do_z[b0] = do[b0]
    ve = synth.ve_inputs(w, layer)
    x, gw, ids, table = ve
    W = w.windows[layer]
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do_z))
    ve_d = tuple(t.cuda() for t in ve)
    o, lse = sa.sa_attn_fwd(qd, kd, vd, window=W, softmax_scale=w.scale, eps=w.eps, ve=ve_d)
    dq, dk, dv, dve, dw, dx32 = sa.sa_attn_bwd(qd, kd, vd, o, lse, dod, window=W, softmax_scale=w.scale,
                                               eps=w.eps, ve=ve_d)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    dw_ref = torch.zeros((w.Hkv, 32), dtype=torch.float64)
    dx_ref = torch.zeros((w.T, 32), dtype=torch.float64)
    dve_ref = torch.zeros((w.T, w.Hkv, w.D), dtype=torch.float64)
    for g in range(w.Hkv):
        hs = slice(g * G, (g + 1) * G)
        ve_g = (x[b0:b0 + 1, :, :32], gw[g:g + 1], ids[b0:b0 + 1], table[:, g * w.D:(g + 1) * w.D])
        _, _, _, dve_g, dw_g, dx_g = oracle.attn_backward(q[b0:b0 + 1, :, hs], k[b0:b0 + 1, :, g:g + 1],
                                                          v[b0:b0 + 1, :, g:g + 1], do[b0:b0 + 1, :, hs], W,
                                                          w.scale, eps=w.eps, ve=ve_g)
        dw_ref[g] = dw_g[0]
        dx_ref += dx_g[0]
        dve_ref[:, g] = dve_g[0, :, 0]
    e_w = rel_l2(dw.cpu(), dw_ref)
    e_x = rel_l2(dx32[b0].cpu(), dx_ref)
    e_ve = rel_l2(dve[b0].cpu(), dve_ref)
    log(f"  dw rel-L2 {e_w:.3e}  dx32 rel-L2 {e_x:.3e}  dve rel-L2 {e_ve:.3e}")
    assert e_w <= 5e-2 and e_x <= 5e-2 and e_ve <= 5e-2
    others = torch.ones(w.B, dtype=torch.bool)
    others[b0] = False
    for name, t in (("dx32", dx32), ("dve", dve), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert not bool(t[others.cuda()].float().abs().max() > 0), f"{name} nonzero outside batch row {b0}"
