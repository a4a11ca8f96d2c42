// Prologue of the two-warp-group forward: per call, every key row is RMS
// normed once ([post] QK-norm passage; [guide] 8.2.1) and written as k_hat in
// the layout of k, and the value rows of each (batch, KV head) are written
// transposed, as v_t[b][g][d][t] with the key axis padded with zeros to a
// multiple of 64. With value embeddings the value rows are mixed first
// (v + gate * embedding, ve_common.h). With rotary tables the key rows are turned first (pairs
// of dimensions i and i + D/2 by the angle of the row's position; the norm
// is unchanged by the turn). After it, the attention kernel's key and value tiles are
// plain copies that go straight from memory into LDS, and both are read
// there with 16-byte reads (the value operand of P.V runs along keys).
// HBM-bound: each k and v element is read once and written once.
#include "sa_common.h"
#include "sa_kernels.h"
#include "ve_common.h"

namespace sa {

template <int D>
__global__ void __launch_bounds__(256) kv_prep_kernel(KvPrepParams p) {
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;   // rows per pass of the workgroup
  // LDS pitch of the staged value tile: D + 2 elements is an odd number of
  // 4-byte words, so the 2-byte column reads of the transposed write (keys
  // 8c + 2j, c = 0..7, at one column) fall on distinct banks
  constexpr int VP = D + 2;
  __shared__ __attribute__((aligned(16))) bf16 vs[64 * VP];

  const int t0 = blockIdx.x * 64;
  const int bg = blockIdx.y;  // b * Hkv + g
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int sub = threadIdx.x % CPR;
  const bool ve_on = p.ve.x != nullptr;
  const auto rt = make_rsrc(p.ve.table, p.ve_table_bytes);

  // every row's loads first (the stores below could alias them for the
  // compiler, which would then keep each pass's loads behind the previous
  // pass's stores)
  constexpr int NP = 64 / RPP;  // passes over the workgroup's 64 rows
  u32x4 kws[NP], vws[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = t0 + threadIdx.x / CPR + i * RPP;
    kws[i] = vws[i] = u32x4{0u, 0u, 0u, 0u};
    if (t < p.T) {
      const long off = (((long)b * p.T + t) * p.Hkv + g) * D + 8 * sub;
      kws[i] = ld16((const bf16*)p.k + off);
      vws[i] = ld16((const bf16*)p.v + off);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = threadIdx.x / CPR + i * RPP;
    const int t = t0 + r;
    const bool in = t < p.T;
    const long off = (((long)b * p.T + (in ? t : 0)) * p.Hkv + g) * D + 8 * sub;
    const u32x4 kw = kws[i];
    u32x4 vw = vws[i];
    if (in && ve_on) {
      // value-embedding gate: v + 2 sigmoid(x[:32] . w[g]) table[id][g]
      const long row = (long)b * p.T + t;
      const float gt = ve_gate_of(p.ve, row, g);
      float vv[8], ee[8];
      unpack8(vw, vv);
      unpack8(ve_chunk(p.ve, rt, p.ve_table_bytes, row, p.Hkv, D, g, sub), ee);
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = __builtin_fmaf(gt, ee[e], vv[e]);
      vw = pack8(vv);
    }
    float x[8];
    unpack8(kw, x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    const float rs = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
    if (p.rope.cos != nullptr) {
      // the partner chunk (the other half of the row) is CPR/2 lanes away
      float xp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xp[e] = __shfl_xor(x[e], CPR / 2);
      const long tr = (long)(in ? t : 0) * p.rope.stride + 8 * (sub % (CPR / 2));
      rope8(x, xp, p.rope.cos + tr, p.rope.sin + tr, sub >= CPR / 2, false);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= rs;
    if (in) st16((bf16*)p.khat + off, pack8(x));
    uint32_t* vrow = (uint32_t*)(vs + r * VP + 8 * sub);  // 4-byte aligned at this pitch
#pragma unroll
    for (int e = 0; e < 4; ++e) vrow[e] = vw[e];  // rows past T stay zero
  }
  __syncthreads();

  // transposed write: thread -> (d, 8-key chunk c); 128 contiguous bytes per d row
  const unsigned short* vu = (const unsigned short*)vs;
  const int c = threadIdx.x % 8;
  for (int d = threadIdx.x / 8; d < D; d += 32) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)vu[(8 * c + 2 * j) * VP + d] | ((uint32_t)vu[(8 * c + 2 * j + 1) * VP + d] << 16);
    st16((bf16*)p.vt + ((long)bg * D + d) * p.Tp + t0 + 8 * c, w);
  }
}

hipError_t launch_kv_prep(const KvPrepParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev) {
  const dim3 grid((unsigned)(p.Tp / 64), (unsigned)(p.B * p.Hkv));
  if (head_dim == 128)
    hipExtLaunchKernelGGL((kv_prep_kernel<128>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((kv_prep_kernel<64>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

}  // namespace sa
