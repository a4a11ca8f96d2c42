// Kernel parameter blocks and host-side launchers (internal to libsa_attn.so).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Rotary embedding tables: fp32, row t (position t) at cos + t * stride and
// sin + t * stride, head_dim / 2 entries; dimension i < D/2 pairs with
// i + D/2. cos == nullptr: no rotation.
struct Rope {
  const float* cos;
  const float* sin;
  int stride;
};

// Value-embedding gate inputs (x == nullptr: none): x bf16 rows of x_stride
// elements (the first 32 read), w bf16 [Hkv][32], ids int32 [B*T], table
// bf16 [vocab][Hkv*D] (read through a buffer of table_bytes: ids past it read zeros).
struct VeParams {
  const void* x;
  long x_stride;
  const void* w;
  const int32_t* ids;
  const void* table;
};
constexpr int kVeRows = 32;  // rows per workgroup of the gate's passes (and per partial sum of dw)
constexpr int kVeMaxHeads = 16;  // KV heads the value-embedding gate supports

struct VePrepParams {
  VeParams ve;
  const void* v;
  void* v_mixed;   // bf16 [rows, Hkv, D]
  float* gate;     // fp32 [rows, Hkv]
  long rows;       // B * T
  int Hkv;
  uint32_t table_bytes;
};

struct VeBwdParams {
  VeParams ve;
  const void* dv;      // dL/dv' (bf16 [rows, Hkv, D])
  const float* gate;   // as written by ve_prep
  void* dve;           // bf16 [rows, Hkv, D]
  float* dx32;         // fp32 [rows, 32]
  float* part;         // fp32 [Hkv * 32, ceil(rows / kVeRows)] (workspace): per (head, channel), the blocks' partials
  float* dw;           // fp32 [Hkv, 32]
  long rows;
  int Hkv;
  uint32_t table_bytes;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* khat;      // normed k rows [B, T, Hkv, D] (norm pass output)
  const void* v;
  const void* vrows;     // value rows the attention runs on [B, T, Hkv, D]: v, or v' with value embeddings
  void* o;
  float* lse;
  int B, T, Hq, Hkv, G;  // G = Hq / Hkv
  int window;            // -1 = full causal (already normalised by the host)
  float c1;              // softmax_scale * log2(e): logits in the base-2 domain
  float c2;              // fixed row maximum (base 2) when the logits are bounded
  float eps;
  int nqb;               // number of query blocks (128 rows; 256 with pair_rows)
  int nsub;              // workgroups per (batch, KV head, query block) = G / heads-per-workgroup
  int pair_rows;         // two-group kernels: 0 = the two warp groups take the same 128 rows of two
                         // query heads; 1 = they take alternate 32-row slices of 256 rows of one head (odd G)
  int nwg;               // workgroups of a persistent launch (one per compute unit)
  Rope rope;             // rotary tables for q (k is turned by the prologue kernel)
};


struct BwdParams {
  const void* q;
  const void* k;
  const void* khat;   // normed k rows [B, T, Hkv, D] (k itself without the norm)
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // fp32 [B, Hq, T], written by the dQ kernel
  float* lse2;    // fp32 [B, Hq, T]: the forward's LSE times log2(e), written by the dQ kernel
  void* qhat;     // bf16 [B, T, Hq, D]: normed q rows written by the dQ kernel (q itself without the norm)
  const float* rstd_k;  // fp32 [B, T, Hkv]: 1/rms of the k rows, written by the norm pass (with the QK-norm)
  int B, T, Hq, Hkv, G;
  int window;
  float scale;
  float c1;       // scale * log2(e)
  float eps;
  int nqb;        // number of query blocks (dQ kernel; 128 rows, 256 with pair_rows)
  int nsub;       // dQ workgroups per (batch, KV head, query block)
  int pair_rows;  // as in FwdParams
  int nkb;        // number of 128-key blocks (dK/dV kernel)
  int nwg;        // workgroups of a persistent launch (one per compute unit)
  Rope rope;      // rotary tables: q_hat is written turned, dq and dk are turned back
};

struct NormParams {
  const void* x;
  void* y;
  float* rstd;
  int64_t rows;
  float eps;
  Rope rope;   // optional: rows are [B, T, H] head rows, turned by position t = (row / H) % T
  int H, T;
};

// Batched bf16 GEMM of the polar-express iteration: per matrix b,
// C[b] = alpha A[b] op(B[b]) + beta C0[b], A [M][K], op(B) = B^T with B
// [N][K] or B with B [K][N]; C, C0 [M][N]; M, N multiples of 128, K of 64.
struct GemmParams {
  const void* a;
  const void* b;
  const void* c0;  // nullptr: beta ignored
  void* c;
  int M, N, K;
  float alpha, beta;
  int sym;         // C is symmetric (M == N): only tiles on or above the diagonal are computed, each stored mirrored too
  int splits;      // K in this many equal ranges (0 or 1: none); fp32 partial tiles in part, summed by a second kernel
  float* part;     // batch * splits * (computed tiles) * 128 * 128 floats
  const float* nsum;  // optional: per matrix nsum_n partial sums whose total is ||G||_F^2 for an operand G;
                      // alpha is then multiplied by s^npow_a and beta by s^npow_b, s = 1 / (||G||_F + neps)
  int nsum_n;
  int npow_a, npow_b;
  float neps;
  float* trace;       // optional (symmetric, 128 x 128 tiles): per matrix 4 (M / 128) partial sums of the
                      // diagonal of the unscaled product, one per 32 x 32 diagonal block, in block order
};
// Partial sums per matrix of the diagonal that a symmetric GEMM writes to GemmParams::trace.
__host__ __device__ inline int gemm_trace_parts(int M) { return 4 * (M / 128); }
// Tiles of C that a GEMM computes (all, or those on and above the diagonal; tile_m x tile_n
// tiles, square when symmetric).
__host__ __device__ inline int gemm_tiles(int M, int N, int sym, int tile_m = 128, int tile_n = 128) {
  const int tm = M / tile_m, tn = N / tile_n;
  return sym ? tm * (tm + 1) / 2 : tm * tn;
}

// Optional events of a kernel launch (benchmarking hook), attached to the kernel's own
// dispatch (hipExtLaunchKernelGGL), so their elapsed time is the kernel's duration.
struct TimingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launchers return the first HIP error seen (hipGetLastError() after the launches).
hipError_t launch_fwd(const FwdParams& p, int head_dim, int heads_per_wg, bool qk_norm, bool fixed_max,
                      hipStream_t stream, const TimingEvents& ev);
// Two-warp-group forward with bounded logits (any query-heads-per-KV-head ratio; p.pair_rows for odd ones).
hipError_t launch_fwd_pp(const FwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev);
// Two-warp-group dQ kernel (reads p.khat; p.pair_rows for an odd query-heads-per-KV-head ratio).
hipError_t launch_bwd_dq_pp(const BwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev);
// dK/dV kernel whose two warp groups (per-key state split by role) alternate on the matrix cores
// (any query-heads-per-KV-head ratio).
hipError_t launch_bwd_dkdv_pp(const BwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev);
// With ve: the same launch also writes the value-embedding mix v' and the gate.
hipError_t launch_qknorm(const NormParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev,
                         const VePrepParams* ve = nullptr);
// Polar-express pieces: GEMM (b_kn: B given as [K][N]; tile: 128 (128 x 128), 96 (96 x 128, b_kn
// only, unsplit), 64 (64 x 64, not b_kn, unsplit) or 192 (192 x 192, unsplit; M, N multiples of 192,
// K of 32); trace only with 128; a_kn: A given as [K][M] too, with b_kn and tile 128).
hipError_t launch_gemm(const GemmParams& p, bool b_kn, int batch, hipStream_t stream, int tile = 128,
                       bool a_kn = false);
// Value-embedding gate backward: dve, dx32 and dw from dL/dv' (v' and g come from the norm pass).
hipError_t launch_ve_bwd(const VeBwdParams& p, int head_dim, hipStream_t stream);

}  // namespace sa
