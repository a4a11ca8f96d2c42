"""fp64 CPU oracle for QK-normed, grouped-query, sliding-window causal attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the entry module and
the CPU-baseline leg of the benchmark use it. It shares no code with the HIP
path (no kernels, headers, helpers or constants); the only common module is
the seeded input generator ``synth``.

What it computes is the plain definition, in float64, with no blocking, no
fusion and no rounding:

  1. weightless RMS norm of every q and k head row over head_dim
     x_hat = x / sqrt(mean(x^2) + eps)
  2. grouped-query head map: query head h reads KV head floor(h / (Hq/Hkv))
  3. logits S_ij = scale * <q_hat_i, k_hat_j>
  4. band: key j is visible to query i iff 0 <= i - j <= W, or j <= i when
     W = -1 (full causal)
  5. softmax over the band, O_i = sum_j P_ij v_j, LSE_i = log sum_j exp(S_ij)
  6. backward of 1-5 with respect to the raw q, k, v
  optional: the rotary position embedding of q and k rows (tables of cos and
  sin given per position), applied before step 1
  optional: the value-embedding gate of the value rows (below), applied to v
  before step 5

Sources (cited by page title and section):
  [post]   The social post that walks through autoresearch's train.py
           (Spanish, French, German and Czech editions of discover post
           71151920174080); its paragraph on the model: RMSNorm on queries
           and keys just before the attention dot product (QK-norm), the
           "SSSL" pattern of three sliding-window layers with a window of
           half the sequence length followed by one full causal layer, the
           8-layer map and the forced-global last layer.
  [guide]  "autoresearch Administrator & Developer Guide": section 3.4
           (WINDOW_PATTERN row: last layer always overridden to L),
           section 6.3 (techniques table: sliding windows, GQA),
           section 8.2.1 (model table: RMSNorm via F.rms_norm, GQA with
           n_kv_head <= n_head, per-layer window from WINDOW_PATTERN).

Readings where the pages are silent (each one is listed in the design notes):
  - window boundary: key j with 0 <= i - j <= W is visible, i.e. W + 1 keys
    counting the query's own position; W >= T - 1 is full causal;
  - norm: weightless, over head_dim, eps = 1e-6 inside the square root;
  - GQA map: contiguous groups, h -> floor(h / G);
  - no attention-logit softcap, no dropout, no document mask;
  - LSE in natural log; gradients are with respect to the raw (un-normed)
    q and k;
  - rotary embedding ([guide] 8.2.1 lists precomputed rotary tables and no
    formula): dimension i < D/2 pairs with i + D/2 and both turn by the angle
    theta[t, i] of the row's position t, taken from caller-given cos/sin
    tables; the default tables use theta[t, i] = t * 10000^(-2i/D). The
    rotation is applied to q and k before their norm (it preserves each
    row's length, so the two commute).

Every helper below is a module attribute so a test can replace one with a
planted mistake and show that the pins catch it.

Parity status: every public function here is pinned by the CPU tests
(closed forms, library routines the pages name, finite differences,
brute force); none is "parity unpinned".
"""

from __future__ import annotations

import math

import torch

F64 = torch.float64


# ---------------------------------------------------------------- schedule

def sssl_windows(n_layer: int, seq_len: int, pattern: str = "SSSL") -> list:
    """Per-layer window list for a pattern of 'S' (local) / 'L' (global) letters.

    [post] model paragraph: the pattern repeats over the layers, 'S' layers
    use a sliding window of half the sequence length, 'L' layers are full
    causal, and the last layer is forced to be global whatever the pattern.
    [guide] 3.4, WINDOW_PATTERN row. Returns -1 for full causal.
    """
    if not pattern or any(c not in "SL" for c in pattern.upper()):
        raise ValueError(f"pattern must be a non-empty string of S/L, got {pattern!r}")
    pattern = pattern.upper()
    out = []
    for layer in range(n_layer):
        letter = pattern[layer % len(pattern)]
        if layer == n_layer - 1:
            letter = "L"
        out.append(-1 if letter == "L" else seq_len // 2)
    return out


# ---------------------------------------------------------------- mask

def band_mask(T: int, window: int) -> torch.Tensor:
    """[T, T] bool, entry (i, j) true iff key j is visible to query i.

    Causal (j <= i) and, for window >= 0, within the window (i - j <= window).
    [post] model paragraph (banded attention matrix of the local layers);
    [guide] 8.2.1 (sliding-window attention row).
    """
    i = torch.arange(T).view(T, 1)
    j = torch.arange(T).view(1, T)
    visible = j <= i
    if window >= 0:
        visible = visible & ((i - j) <= window)
    return visible


# ---------------------------------------------------------------- norm

def rms_norm(x: torch.Tensor, eps: float):
    """Weightless RMS norm over the last dim: returns (x_hat, r), r = (ms + eps)^-1/2.

    [post] model paragraph (RMSNorm on queries and keys just before the
    attention dot product); [guide] 8.2.1 (RMSNorm via F.rms_norm, no weight).
    """
    x = x.to(F64)
    ms = (x * x).mean(dim=-1, keepdim=True)
    r = 1.0 / torch.sqrt(ms + eps)
    return x * r, r


def rms_norm_backward(x_hat: torch.Tensor, r: torch.Tensor, dx_hat: torch.Tensor) -> torch.Tensor:
    """Gradient through x_hat = r * x, r = (mean(x^2) + eps)^-1/2.

    d x_hat_a / d x_b = r * delta_ab - r^3 * x_a * x_b / D, hence
    dx = r * (dx_hat - x_hat * <dx_hat, x_hat> / D).
    """
    D = x_hat.shape[-1]
    return r * (dx_hat - x_hat * (dx_hat * x_hat).sum(dim=-1, keepdim=True) / D)


# ---------------------------------------------------------------- rotary embedding

def rope_angles(T: int, D: int, base: float = 10000.0) -> torch.Tensor:
    """[T, D/2] float64 angles theta[t, i] = t * base^(-2i/D).

    [guide] 8.2.1 (rotary embeddings, precomputed tables); the frequency
    ladder is the reading listed in the module docstring.
    """
    t = torch.arange(T, dtype=F64).view(T, 1)
    i = torch.arange(D // 2, dtype=F64).view(1, D // 2)
    return t * torch.pow(torch.tensor(base, dtype=F64), -2.0 * i / D)


def rope_tables(T: int, D: int, base: float = 10000.0):
    """(cos, sin) [T, D/2] float64 of rope_angles."""
    a = rope_angles(T, D, base)
    return torch.cos(a), torch.sin(a)


def rope_rotate(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotary embedding of x [B, T, H, D]: row (b, t, h) turns each pair
    (x_i, x_{i+D/2}) by the angle of table row t:
      y_i = x_i cos - x_{i+D/2} sin,   y_{i+D/2} = x_i sin + x_{i+D/2} cos.
    cos and sin have at least T rows of D/2 entries.
    """
    x = x.to(F64)
    T, D = x.shape[1], x.shape[-1]
    c = cos[:T].to(F64).view(1, T, 1, D // 2)
    s = sin[:T].to(F64).view(1, T, 1, D // 2)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)


def rope_rotate_back(y: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Transpose (inverse) of rope_rotate: the gradient map of the rotation."""
    y = y.to(F64)
    T, D = y.shape[1], y.shape[-1]
    c = cos[:T].to(F64).view(1, T, 1, D // 2)
    s = sin[:T].to(F64).view(1, T, 1, D // 2)
    y1, y2 = y[..., : D // 2], y[..., D // 2:]
    return torch.cat([y1 * c + y2 * s, -y1 * s + y2 * c], dim=-1)


# ---------------------------------------------------------------- value embeddings

def ve_layers(n_layer: int) -> list:
    """Layers that carry value embeddings: alternating, the last always included
    ([guide] 8.2.1)."""
    return [i for i in range(n_layer) if (n_layer - 1 - i) % 2 == 0]


def ve_gate(x32: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """gate [B, T, Hkv] = 2 sigmoid(x[..., :32] W^T): [guide] 8.2.1, the value-embedding
    gate (a bias-free linear map of the first 32 channels to one value per KV head)."""
    z = x32.to(F64) @ w.to(F64).transpose(0, 1)
    return 2.0 * torch.sigmoid(z)


def ve_mix(v: torch.Tensor, x32: torch.Tensor, w: torch.Tensor, ids: torch.Tensor, table: torch.Tensor):
    """v + gate[..., None] * ve with ve = table[ids] viewed [B, T, Hkv, D] ([guide] 8.2.1)."""
    B, T, Hkv, D = v.shape
    ve = table.to(F64)[ids.long()].view(B, T, Hkv, D)
    return v.to(F64) + ve_gate(x32, w).unsqueeze(-1) * ve


def ve_backward(dv_mixed, x32, w, ids, table):
    """Gradients of the mix, given dL/dv' for v' = v + g ve, g = 2 sigmoid(z), z = x32 W^T:
    dv = dv', dve = g dv', dg = <dv', ve> over D, dz = dg g (1 - g/2),
    dW = sum_{b,t} dz^T x32, dx32 = dz W. Returns (dve [B,T,Hkv,D], dW [Hkv,32], dx32 [B,T,32])."""
    B, T, Hkv, D = dv_mixed.shape
    dvm = dv_mixed.to(F64)
    ve = table.to(F64)[ids.long()].view(B, T, Hkv, D)
    g = ve_gate(x32, w)
    dve = g.unsqueeze(-1) * dvm
    dz = (dvm * ve).sum(-1) * g * (1.0 - g / 2.0)
    dw = torch.einsum("bth,btc->hc", dz, x32.to(F64))
    dx32 = dz @ w.to(F64)
    return dve, dw, dx32


# ---------------------------------------------------------------- heads

def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Grouped-query map: query head h shares KV head floor(h / (Hq / Hkv)).

    [guide] 6.3 and 8.2.1 (grouped-query attention, n_kv_head <= n_head).
    """
    return h // (Hq // Hkv)


def _check_shapes(q, k, v):
    B, T, Hq, D = q.shape
    Bk, Tk, Hkv, Dk = k.shape
    if (Bk, Tk, Dk) != (B, T, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q [B,T,Hq,D], k and v [B,T,Hkv,D] expected")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, T, Hq, Hkv, D


def _normed(q, k, qk_norm, eps, rope=None):
    if rope is not None:
        q = rope_rotate(q, *rope)
        k = rope_rotate(k, *rope)
    if qk_norm:
        q_hat, r_q = rms_norm(q, eps)
        k_hat, r_k = rms_norm(k, eps)
    else:
        q_hat, r_q = q.to(F64), None
        k_hat, r_k = k.to(F64), None
    return q_hat, r_q, k_hat, r_k


def _probs_one_head(q_hat_bh, k_hat_bg, mask, scale):
    """P [T, T] and LSE [T] for one (batch, head): masked softmax of the logits."""
    S = scale * (q_hat_bh @ k_hat_bg.transpose(0, 1))
    S = S.masked_fill(~mask, -math.inf)
    m = S.max(dim=-1, keepdim=True).values
    e = torch.exp(S - m)
    denom = e.sum(dim=-1, keepdim=True)
    P = e / denom
    lse = (m + torch.log(denom)).squeeze(-1)
    return P, lse


# ---------------------------------------------------------------- forward

def attention_probs(q, k, window, scale, qk_norm=True, eps=1e-6, rope=None):
    """Softmax probabilities P [B, Hq, T, T] (zero outside the band)."""
    B, T, Hq, Hkv, D = _check_shapes(q, k, k)
    q_hat, _, k_hat, _ = _normed(q, k, qk_norm, eps, rope)
    mask = band_mask(T, window)
    P = torch.zeros(B, Hq, T, T, dtype=F64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P[b, h], _ = _probs_one_head(q_hat[b, :, h], k_hat[b, :, g], mask, scale)
    return P


def attn_forward(q, k, v, window, scale, qk_norm=True, eps=1e-6, rope=None, ve=None):
    """Forward of the layer: returns (o [B,T,Hq,D], lse [B,Hq,T]) in float64.

    q [B,T,Hq,D], k and v [B,T,Hkv,D] (any float dtype; upcast exactly);
    rope = (cos, sin) tables turn q and k rows first (rope_rotate);
    ve = (x32, w, ids, table) mixes value embeddings into v first (ve_mix).
    """
    B, T, Hq, Hkv, D = _check_shapes(q, k, v)
    q_hat, _, k_hat, _ = _normed(q, k, qk_norm, eps, rope)
    v = v.to(F64) if ve is None else ve_mix(v, *ve)
    mask = band_mask(T, window)
    o = torch.zeros(B, T, Hq, D, dtype=F64)
    lse = torch.zeros(B, Hq, T, dtype=F64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P, lse[b, h] = _probs_one_head(q_hat[b, :, h], k_hat[b, :, g], mask, scale)
            o[b, :, h] = P @ v[b, :, g]
    return o, lse


def attn_forward_rows(q, k, v, rows, window, scale, qk_norm=True, eps=1e-6, with_abs=False):
    """O and LSE of selected query rows of every (batch, head), in float64:
    the forward's definition (masked softmax of the scaled normed logits, then
    the weighted sum of v) evaluated for the rows listed only, so that every
    (batch, head) of a full-size layer can be sampled at small cost.

    rows: 1-D sequence of query positions; returns (o [B, R, Hq, D],
    lse [B, Hq, R]) for the R rows in the order given, and with with_abs also
    the weighted sum of |v| with the same probabilities (the scale of O's
    rounding error when the averaged values have mixed signs).
    """
    B, T, Hq, Hkv, D = _check_shapes(q, k, v)
    rows = torch.as_tensor(rows, dtype=torch.long)
    R = rows.numel()
    q_sel = q[:, rows]
    if qk_norm:
        q_hat, _ = rms_norm(q_sel, eps)
        k_hat, _ = rms_norm(k, eps)
    else:
        q_hat, k_hat = q_sel.to(F64), k.to(F64)
    vv = v.to(F64)
    mask = band_mask(T, window)[rows]  # [R, T]
    o = torch.zeros(B, R, Hq, D, dtype=F64)
    o_abs = torch.zeros(B, R, Hq, D, dtype=F64)
    lse = torch.zeros(B, Hq, R, dtype=F64)
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        S = scale * (q_hat[:, :, h] @ k_hat[:, :, g].transpose(1, 2))  # [B, R, T]
        S = S.masked_fill(~mask, -math.inf)
        m = S.max(dim=-1, keepdim=True).values
        e = torch.exp(S - m)
        denom = e.sum(dim=-1, keepdim=True)
        o[:, :, h] = (e / denom) @ vv[:, :, g]
        if with_abs:
            o_abs[:, :, h] = (e / denom) @ vv[:, :, g].abs()
        lse[:, h] = (m + torch.log(denom)).squeeze(-1)
    return (o, lse, o_abs) if with_abs else (o, lse)


# ---------------------------------------------------------------- backward

def attn_backward(q, k, v, do, window, scale, qk_norm=True, eps=1e-6, rope=None, ve=None):
    """Gradients (dq, dk, dv) of <O, dO> with respect to the raw q, k, v (float64).

    Per (b, h) with g its KV head:
      dV_g   += P^T dO
      dP      = dO V_g^T
      Delta_i = sum_j P_ij dP_ij
      dS      = P * (dP - Delta)
      dq_hat  = scale * dS K_hat_g
      dk_hat_g += scale * dS^T Q_hat
    then the RMS-norm backward maps dq_hat, dk_hat to the gradients of the
    rotated rows, and (with rope) the transposed rotation to dq, dk.
    With ve = (x32, w, ids, table) the value rows are the mixed ones and the
    result also holds (dve, dw, dx32) of ve_backward: (dq, dk, dv, dve, dw, dx32).
    """
    B, T, Hq, Hkv, D = _check_shapes(q, k, v)
    q_hat, r_q, k_hat, r_k = _normed(q, k, qk_norm, eps, rope)
    v = v.to(F64) if ve is None else ve_mix(v, *ve)
    do = do.to(F64)
    mask = band_mask(T, window)
    dq_hat = torch.zeros(B, T, Hq, D, dtype=F64)
    dk_hat = torch.zeros(B, T, Hkv, D, dtype=F64)
    dv = torch.zeros(B, T, Hkv, D, dtype=F64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            P, _ = _probs_one_head(q_hat[b, :, h], k_hat[b, :, g], mask, scale)
            dO = do[b, :, h]
            dv[b, :, g] += P.transpose(0, 1) @ dO
            dP = dO @ v[b, :, g].transpose(0, 1)
            delta = (P * dP).sum(dim=-1, keepdim=True)
            dS = P * (dP - delta)
            dq_hat[b, :, h] = scale * (dS @ k_hat[b, :, g])
            dk_hat[b, :, g] += scale * (dS.transpose(0, 1) @ q_hat[b, :, h])
    if qk_norm:
        dq = rms_norm_backward(q_hat, r_q, dq_hat)
        dk = rms_norm_backward(k_hat, r_k, dk_hat)
    else:
        dq, dk = dq_hat, dk_hat
    if rope is not None:
        dq = rope_rotate_back(dq, *rope)
        dk = rope_rotate_back(dk, *rope)
    if ve is not None:
        return (dq, dk, dv) + ve_backward(dv, *ve)
    return dq, dk, dv


def attn_backward_delta(o, do):
    """Delta_i = <dO_i, O_i> per (b, h, i) as [B, Hq, T]; equal to sum_j P_ij dP_ij."""
    return (o.to(F64) * do.to(F64)).sum(dim=-1).permute(0, 2, 1).contiguous()


def qknorm(x, eps=1e-6):
    """Standalone norm of [rows, D] rows: returns (y, rstd) with rstd [rows]."""
    y, r = rms_norm(x, eps)
    return y, r.squeeze(-1)
