/*
 * sa_attn.h - C ABI of libsa_attn.so: QK-normed, grouped-query, sliding-window
 * causal attention (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * The layer it implements is the attention of the small GPT trainer that the
 * following pages describe:
 *   [post]  the social post walking through autoresearch's train.py (Spanish,
 *           French, German and Czech editions of discover post
 *           71151920174080), paragraph on the model: RMSNorm on queries and
 *           keys just before the attention dot product ("QK-norm"); the "SSSL"
 *           pattern of three sliding-window layers (window = half the sequence
 *           length) and one full causal layer, repeating, last layer global.
 *   [guide] "autoresearch Administrator & Developer Guide", section 8.2.1
 *           (model table: RMSNorm via F.rms_norm, grouped-query attention with
 *           n_kv_head <= n_head, per-layer sliding window) and section 6.3.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory) unless a
 *     parameter says otherwise. The caller allocates and owns every buffer,
 *     including the backward workspace; the library never allocates, frees,
 *     synchronises or prints.
 *   - Tensors are contiguous, row-major, innermost dimension last:
 *       q, o, dout, dq : bf16 [B, T, Hq,  D]
 *       k, v, dk, dv   : bf16 [B, T, Hkv, D]
 *       lse            : fp32 [B, Hq, T]   natural-log log-sum-exp of the
 *                                          scaled logits over the band
 *     bf16 is the IEEE-754 binary32 upper half (bfloat16), RNE rounding.
 *   - D (head_dim) is 64 or 128. Hq must be a multiple of Hkv; query head h
 *     reads KV head floor(h / (Hq / Hkv)) (contiguous groups).
 *   - window: -1 = full causal. window >= 0: key j is visible to query i iff
 *     0 <= i - j <= window (window + 1 keys counting the query itself). Any
 *     window >= T - 1 is treated as full causal.
 *   - qk_norm != 0 applies the weightless RMS norm
 *       x_hat = x / sqrt(mean(x^2) + eps)
 *     to every q and k head row (over D) before the logits
 *     S_ij = softmax_scale * <q_hat_i, k_hat_j>; qk_norm = 0 uses q and k
 *     as given. Gradients are always with respect to the raw q, k, v.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it; nothing blocks the host.
 *   - Errors: every argument is validated before anything is launched, so an
 *     error return means nothing was enqueued. Faults inside a kernel surface
 *     at the caller's next synchronisation, as with any stream operation.
 *   - Thread safety: no mutable global state (the benchmarking hook below is
 *     per host thread); concurrent calls on different streams are safe.
 */
#ifndef SA_ATTN_H
#define SA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,       /* a size <= 0, Hq % Hkv != 0, window < -1, a non-finite scale or eps,
                             eps < 0, or (T+256)*Hq*128*2 >= 2^31 (per-batch 32-bit addressing) */
  SA_ERR_UNSUPPORTED = 3, /* head_dim not in {64, 128} */
  SA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  SA_ERR_WORKSPACE = 5,   /* workspace NULL, not 256-byte aligned, or smaller than the *_workspace_bytes() size */
  SA_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} sa_status;

/* Version of this ABI (bumped on any incompatible change). */
int sa_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* sa_status_string(int status);

/*
 * sa_qknorm - standalone weightless RMS norm of `rows` rows of length head_dim.
 *   [post] QK-norm passage; [guide] 8.2.1 (RMSNorm via F.rms_norm, no weight).
 *   x    : bf16 [rows, head_dim] input (e.g. q or k viewed as [B*T*H, D]).
 *   y    : bf16 [rows, head_dim] output, y = x / sqrt(mean(x^2) + eps), RNE.
 *          May alias x (in-place) exactly; partial overlap is not allowed.
 *   rstd : fp32 [rows] output 1/sqrt(mean(x^2)+eps), or NULL to skip it.
 *   rows >= 1, head_dim in {64, 128}. rows = 0 is accepted and does nothing.
 */
sa_status sa_qknorm(const void* x, void* y, float* rstd, int64_t rows, int head_dim, float eps,
                    void* stream);

/*
 * sa_attn_fwd - forward of one attention layer.
 *   [post] model paragraph (QK-norm, sliding-window/full causal layers);
 *   [guide] 8.2.1 (GQA, per-layer window).
 *   Computes, per batch b and query head h with KV head g = h / (Hq/Hkv):
 *     P_i = softmax_j over the band of S_ij,  o_i = sum_j P_ij v_j,
 *     lse_i = log sum_{j in band} exp(S_ij).
 *   q, k, v : inputs (layouts above).  o : bf16 output [B,T,Hq,D].
 *   lse     : fp32 output [B,Hq,T]; required (the backward needs it).
 *   workspace: device buffer of at least sa_attn_fwd_workspace_bytes(...)
 *            bytes, 256-byte aligned. Contents on entry are ignored. With
 *            qk_norm (and the fixed row maximum: |softmax_scale| * head_dim
 *            within its bound) it receives, and keeps on return, the bf16
 *            normed (with rotary tables: turned) k rows [B,T,Hkv,D] and their
 *            fp32 1/rms [B,T,Hkv], and with the value-embedding gate the
 *            bf16 rows v' [B,T,Hkv,D] and the fp32 gate [B,T,Hkv]: the
 *            backward of the same layer can read them back instead of
 *            recomputing them (sa_attn_bwd_ex's fwd_workspace). Otherwise
 *            the contents on return are unspecified. May be NULL when
 *            qk_norm == 0. Overlapping calls need different workspaces.
 *   Tiles of the band outside every query's window are never loaded.
 */
size_t sa_attn_fwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim);
sa_status sa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int T, int Hq, int Hkv, int head_dim, int window,
                      float softmax_scale, int qk_norm, float eps, void* stream);

/* Bytes of device workspace sa_attn_fwd / sa_attn_bwd need for these sizes (0 if a size is invalid). */
size_t sa_attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim);

/*
 * sa_attn_bwd - backward of sa_attn_fwd with the same arguments.
 *   Recomputes the probabilities from q, k and the forward's lse:
 *     P_ij = exp(S_ij - lse_i),  Delta_i = <dout_i, o_i>,
 *     dS_ij = P_ij (<dout_i, v_j> - Delta_i),
 *     dq_hat_i = scale sum_j dS_ij k_hat_j,  dk_hat_j = scale sum_{h in group} sum_i dS_ij q_hat_i,
 *     dv_j = sum_{h in group} sum_i P_ij dout_i,
 *   then the RMS-norm backward dx = r (dx_hat - x_hat <dx_hat, x_hat> / D).
 *   Two kernels, no atomics: a dQ kernel per query block (it also writes the
 *   normed q rows, Delta and the base-2 LSE into the workspace) and a persistent dK/dV kernel
 *   over the key blocks; the GQA sums over the query heads of a group happen
 *   inside the dK/dV kernel. With qk_norm a norm pass first writes the normed k rows
 *   into the workspace for both kernels.
 *   q, k, v, o, lse, dout : inputs (o and lse as written by sa_attn_fwd).
 *   dq, dk, dv            : bf16 outputs, fully overwritten.
 *   workspace             : device buffer of at least
 *                           sa_attn_bwd_workspace_bytes(B,T,Hq,Hkv,head_dim)
 *                           bytes (the bf16 normed q rows, the fp32 Delta
 *                           rows, the fp32 LSE rows in base 2, the bf16
 *                           normed k rows and their fp32 1/rms), 256-byte
 *                           aligned;
 *                           contents on entry are ignored and on return
 *                           unspecified. Two calls that overlap in time must
 *                           use different workspaces.
 */
sa_status sa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int B, int T, int Hq, int Hkv, int head_dim, int window,
                      float softmax_scale, int qk_norm, float eps, void* stream);

/*
 * sa_attn_bwd_noalloc - sa_attn_bwd for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses that
 *   forbid hipMalloc). Same arguments, semantics and outputs as sa_attn_bwd,
 *   without the workspace: the library uses its own statically allocated
 *   scratch instead (one copy per GPU, sa_attn_bwd_noalloc_max_bytes() =
 *   80 MiB, held until the process ends) and calls no allocating routine.
 *   Sizes whose workspace (sa_attn_bwd_workspace_bytes) exceeds that maximum
 *   return SA_ERR_WORKSPACE without enqueuing anything; the workloads with
 *   B*T = 32768 tokens, Hq = 6, Hkv = 3, D = 128 need 73 MiB. Every call on a
 *   GPU shares that GPU's scratch: calls that overlap in time on one GPU (two
 *   streams, two host threads) race and must be serialised by the caller.
 *   Nothing in the scratch needs to start at zero. SA_ERR_HIP if the
 *   scratch's device address cannot be obtained.
 */
size_t sa_attn_bwd_noalloc_max_bytes(void);
sa_status sa_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv,
                              int B, int T, int Hq, int Hkv, int head_dim, int window,
                              float softmax_scale, int qk_norm, float eps, void* stream);

/*
 * sa_attn_fwd_rope / sa_attn_bwd_rope - sa_attn_fwd / sa_attn_bwd with the
 * rotary position embedding of q and k fused into the kernels.
 *   [guide] 8.2.1 lists rotary embeddings built from precomputed tables and
 *   gives no formula; the standard rotary embedding is taken. Every q and k
 *   head row at position t turns each pair of dimensions (i, i + D/2),
 *   i < D/2, by the angle whose cosine and sine the tables hold:
 *     c = rope_cos[t * rope_stride + i], s = rope_sin[t * rope_stride + i],
 *     y_i = x_i c - x_{i+D/2} s,   y_{i+D/2} = x_i s + x_{i+D/2} c,
 *   and the RMS norm follows (the turn keeps each row's length, so the order
 *   does not change the result). Outputs and lse are those of sa_attn_fwd on
 *   the turned rows; the gradients are with respect to the raw (unturned,
 *   un-normed) q and k. The usual tables hold cos and sin of
 *   t * 10000^(-2i/D).
 *   rope_cos, rope_sin : fp32 DEVICE tables, read only, 16-byte aligned, at
 *                        least T rows of head_dim/2 entries at a row stride
 *                        of rope_stride floats (rope_stride >= head_dim/2, a
 *                        multiple of 4, T * rope_stride * 4 < 2^31). The
 *                        backward must get the same tables as the forward.
 *   Other arguments, workspaces and outputs as for sa_attn_fwd / sa_attn_bwd.
 *   Additional errors: SA_ERR_NULL for a NULL table, SA_ERR_SHAPE for a bad
 *   stride, SA_ERR_ALIGN for a misaligned table, SA_ERR_UNSUPPORTED when
 *   qk_norm == 0, or (forward) when |softmax_scale| * head_dim is too large
 *   for the kernels' fixed row maximum.
 */
sa_status sa_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                           void* workspace, size_t workspace_bytes,
                           int B, int T, int Hq, int Hkv, int head_dim, int window,
                           float softmax_scale, int qk_norm, float eps,
                           const float* rope_cos, const float* rope_sin, int rope_stride, void* stream);
sa_status sa_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes,
                           int B, int T, int Hq, int Hkv, int head_dim, int window,
                           float softmax_scale, int qk_norm, float eps,
                           const float* rope_cos, const float* rope_sin, int rope_stride, void* stream);

/*
 * sa_attn_fwd_ex / sa_attn_bwd_ex - the forward and backward with the
 * optional extras of the trainer's attention, each group all-or-none (NULL
 * pointers: absent):
 *   rotary tables : rope_cos, rope_sin, rope_stride as for sa_attn_fwd_rope;
 *   value-embedding gate ([guide] 8.2.1: alternating layers, the last always,
 *   mix a learned embedding of the token ids into v through a gate of the
 *   first 32 channels of the attention's input):
 *     g[b,t,h] = 2 sigmoid(sum_{c<32} ve_x[b,t,c] ve_w[h,c]),
 *     v'[b,t,h,:] = v[b,t,h,:] + g[b,t,h] ve_table[ve_ids[b,t], h*D : (h+1)*D],
 *   and attention runs on v'. (The gate's linear map has no bias: a reading.)
 *     ve_x       : bf16 DEVICE rows [B*T] of ve_x_stride elements (>= 32, a
 *                  multiple of 8), 16-byte aligned; the first 32 are read.
 *     ve_w       : bf16 [Hkv, 32], 16-byte aligned.
 *     ve_ids     : int32 [B*T]; an id outside [0, ve_vocab) reads a zero row.
 *     ve_table   : bf16 [ve_vocab, Hkv*D], 16-byte aligned,
 *                  ve_vocab*Hkv*D*2 < 2^31.
 *   Backward outputs with the gate (all required then):
 *     dv         : the gradient of the raw v (= that of v', the mix is v + ...).
 *     dve        : bf16 [B, T, Hkv, D], the gradient of the gathered embedding
 *                  rows per position (the table's gradient is their sum into
 *                  the rows ve_ids picks: the caller's embedding backward).
 *     dve_w      : fp32 [Hkv, 32], summed over all positions in a fixed order.
 *     dve_x32    : fp32 [B, T, 32], the gradient of ve_x's first 32 channels.
 *     ve_workspace : at least sa_attn_ve_workspace_bytes(B, T, Hkv, head_dim)
 *                  bytes, 256-byte aligned (v', the gate, partial sums).
 *   Both extras need qk_norm (SA_ERR_UNSUPPORTED otherwise, for the gate with
 *   Hkv > 16, and when
 *   |softmax_scale| * head_dim is too large for the fixed row maximum).
 *   fwd_workspace (backward; optional, NULL: none): the workspace that
 *   sa_attn_fwd / sa_attn_fwd_rope / sa_attn_fwd_ex wrote for this layer,
 *   with the same q, k, v, window, scale, eps, tables and gate inputs, and
 *   not written since; fwd_workspace_bytes its size. The backward then
 *   reads the normed k rows, their 1/rms and (gate) v' and the gate from it
 *   instead of recomputing them, so a trainer that keeps the forward's
 *   workspace per layer saves those passes. Read only; 256-byte aligned, at
 *   least sa_attn_fwd_workspace_bytes(...) bytes (SA_ERR_WORKSPACE);
 *   SA_ERR_UNSUPPORTED when qk_norm == 0 or the scale is beyond the fixed
 *   row maximum (the forward then does not write it).
 *   Other errors as for the plain calls, plus SA_ERR_NULL for a partial group,
 *   SA_ERR_SHAPE for a bad stride or vocabulary, SA_ERR_ALIGN, SA_ERR_WORKSPACE.
 */
sa_status sa_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                         void* workspace, size_t workspace_bytes,
                         int B, int T, int Hq, int Hkv, int head_dim, int window,
                         float softmax_scale, int qk_norm, float eps,
                         const float* rope_cos, const float* rope_sin, int rope_stride,
                         const void* ve_x, int64_t ve_x_stride, const void* ve_w, const int32_t* ve_ids,
                         const void* ve_table, int ve_vocab, void* stream);
size_t sa_attn_ve_workspace_bytes(int B, int T, int Hkv, int head_dim);
sa_status sa_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes,
                         const void* fwd_workspace, size_t fwd_workspace_bytes,
                         int B, int T, int Hq, int Hkv, int head_dim, int window,
                         float softmax_scale, int qk_norm, float eps,
                         const float* rope_cos, const float* rope_sin, int rope_stride,
                         const void* ve_x, int64_t ve_x_stride, const void* ve_w, const int32_t* ve_ids,
                         const void* ve_table, int ve_vocab,
                         void* dve, float* dve_w, float* dve_x32, void* ve_workspace, size_t ve_workspace_bytes,
                         void* stream);

/*
 * sa_polar_express - Muon's orthogonalisation of a stack of bf16 matrices
 * ("autoresearch Administrator & Developer Guide", section 8.2.3): per matrix
 *   X = G / (||G||_F + eps), then for the first `steps` of the five printed
 *   coefficient triples (a, b, c):
 *     A = X X^T (or X^T X for a tall matrix: the smaller square),
 *     B = b A + c A A,  X <- a X + B X (or a X + X B),
 *   out = X. (The guide does not show the initial scaling; dividing by the
 *   Frobenius norm bounds every singular value by 1, the range the
 *   coefficients are made for.)
 *   g, out    : bf16 [batch, rows, cols], contiguous, 16-byte aligned; out
 *               fully overwritten (must not overlap g).
 *   rows, cols: multiples of 128 (SA_ERR_UNSUPPORTED otherwise); one matrix
 *               below 2^31 bytes; batch <= 65535 and batch * (rows / 128) *
 *               (cols / 128) < 2^20 (SA_ERR_SHAPE otherwise).
 *   steps     : 1..5 (5 in the trainer); eps >= 0 (the trainer's guard is tiny).
 *   workspace : at least sa_polar_express_workspace_bytes(batch, rows, cols)
 *               bytes, 256-byte aligned (two copies of X, A and B, partial
 *               sums of the first Gram product's diagonal (||G||_F^2), fp32
 *               partial tiles of the products whose K is split); contents
 *               unspecified.
 *   Arithmetic: bf16 MFMA operands with fp32 accumulation; X, A and B are
 *   stored as bf16 between the products, as a bf16 optimizer step keeps them.
 *   The result depends only on its own matrix: matrices of a stack are
 *   independent.
 */
size_t sa_polar_express_workspace_bytes(int batch, int rows, int cols);
/* MFMA FLOP that sa_polar_express executes for these arguments (the symmetric
 * products compute only their tiles on and above the diagonal, so this is
 * below the full-product count 5 (4 m^2 n + 2 m^3) per matrix); 0 for
 * arguments it would reject. Launches nothing; the tiles it counts depend on
 * the current device's compute units (128 x 128 tiles without a device). */
double sa_polar_express_executed_flops(int batch, int rows, int cols, int steps);
sa_status sa_polar_express(const void* g, void* out, void* workspace, size_t workspace_bytes,
                           int batch, int rows, int cols, int steps, float eps, void* stream);

/* Kernels that sa_set_timing_events can bracket. */
enum {
  SA_KERNEL_FWD = 0,       /* attention kernel of sa_attn_fwd */
  SA_KERNEL_BWD_DQ = 1,    /* dQ kernel of sa_attn_bwd */
  SA_KERNEL_BWD_DKDV = 2,  /* dK/dV kernel of sa_attn_bwd */
  SA_KERNEL_FWD_KNORM = 3, /* key-norm pass of sa_attn_fwd (QK-norm, bounded logits) */
  SA_KERNEL_BWD_KNORM = 4  /* key-norm pass of sa_attn_bwd (QK-norm, no fwd_workspace) */
};

/*
 * sa_set_timing_events - benchmarking hook (not part of the computation).
 *   While set, every later sa_attn_fwd / sa_attn_bwd call (and their _ex
 *   and _noalloc forms) made FROM THE CALLING HOST THREAD that runs the
 *   kernel named by `kernel` (one of the SA_KERNEL_ ids above) attaches
 *   `start` and `stop` to that kernel's own dispatch on its stream
 *   (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is the
 *   kernel's duration, without the gaps of separate event packets. start/stop are hipEvent_t handles
 *   passed as void*, created and owned by the caller; pass NULL, NULL to clear.
 *   Returns SA_ERR_SHAPE for an unknown kernel id, SA_ERR_NULL if exactly one
 *   of start/stop is NULL.
 */
sa_status sa_set_timing_events(int kernel, void* start, void* stop);

/*
 * sa_set_max_workgroups - testing hook (not part of the computation).
 *   The attention kernels run persistently: one workgroup per compute unit,
 *   each taking a fixed share of the work items (query blocks or key blocks).
 *   While n > 0, every later sa_attn_fwd / sa_attn_bwd call made FROM THE
 *   CALLING HOST THREAD launches at most n workgroups, so that small problems
 *   can exercise workgroups that process many items in a row. n = 0 restores
 *   the default (one per compute unit). Results do not depend on n.
 *   Returns SA_ERR_SHAPE for n < 0.
 */
sa_status sa_set_max_workgroups(int n);

#ifdef __cplusplus
}
#endif

#endif /* SA_ATTN_H */
