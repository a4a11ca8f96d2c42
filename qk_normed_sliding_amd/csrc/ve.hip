// Value-embedding gate of the value rows ("autoresearch Administrator &
// Developer Guide", section 8.2.1: alternating layers, the last always, mix a
// learned embedding of the token ids into v):
//   g[b,t,h] = 2 sigmoid(sum_c x[b,t,c] w[h,c]), c < 32,
//   v'[b,t,h,:] = v[b,t,h,:] + g[b,t,h] ve[b,t,h,:],  ve = table[ids[b,t]] viewed [Hkv, D].
// The forward's norm pass writes v' and g once (qknorm.hip) into its workspace and
// runs the attention on v'; the backward reads them back from there (or
// writes them itself without the forward's workspace), runs its kernels on
// v', then maps dL/dv' to the embedding, gate and input gradients:
//   dve = g dv',  dz = <dv', ve> g (1 - g/2),  dx32 = dz w,  dw = sum_{b,t} dz^T x32,
// in one pass per block of rows (dz stays in LDS), dw as fixed-order partial
// sums per block and one reduction.
// dv (the raw v's gradient) is dv' itself. Embedding rows are read through a
// buffer descriptor over the table: an id past the table reads zeros.
#include "sa_common.h"
#include "sa_kernels.h"
#include "ve_common.h"

namespace sa {

// Chunk tasks per pass of the backward's streaming loop: CPR lanes per (row,
// head), one 16-byte chunk each; the workgroup covers kVeRows rows, all heads
// (pairs rh0 .. rh0 + npair, pair i = (row r0 + i / H, head i % H)), U passes
// per group, whose loads are all issued before the first result is used (ids,
// rows and gates first, then the embedding rows the ids select).
template <int D>
struct VeStream {
  static constexpr int CPR = D / 8;
  static constexpr int PPP = 256 / CPR;     // pairs per pass
  static constexpr int U = (kVeRows * 3 + PPP - 1) / PPP;  // passes per group (one group at 3 heads)
};

// The backward of the gate, per block of kVeRows rows, in one pass:
//  1. dve = g dv' per chunk, and dz = <dv', ve> g (1 - g/2) per (row, head)
//     (the dot summed over the pair's lanes) into LDS;
//  2. dx32[row][c] = sum_h dz[row][h] w[h][c];
//  3. the block's partial dw[h][c] = sum_row dz[row][h] x[row][c]: thread
//     (j, c) sums rows j, j + 8, ..., then the 8 row groups are added in
//     order, and the sum is stored at part[(h * 32 + c) * nblk + block] (all
//     blocks of one (h, c) contiguous, for the reduction; fixed order
//     throughout: deterministic).
template <int D>
__global__ void __launch_bounds__(256) ve_bwd_kernel(VeBwdParams p, int nblk) {
  using S = VeStream<D>;
  static_assert(4 * kVeRows <= 256 && kVeRows % 8 == 0, "one 16-byte chunk of x per thread");
  __shared__ float xs[kVeRows][33];
  __shared__ float zs[kVeRows * kVeMaxHeads];  // dz of pair i (row i / H, head i % H)
  __shared__ float wsh[kVeMaxHeads][32];
  __shared__ float acc[8][kVeMaxHeads][32];
  const int tid = threadIdx.x;
  const int H = p.Hkv;
  const long r0 = (long)blockIdx.x * kVeRows;
  const int nr = (int)min((long)kVeRows, p.rows - r0);
  const long rh0 = r0 * H;
  const int npair = nr * H;
  // the block's x rows (first 32 channels), used after the stream
  u32x4 xrow = {0u, 0u, 0u, 0u};
  if ((tid >> 2) < min(nr, kVeRows)) xrow = ld16((const bf16*)p.ve.x + (r0 + (tid >> 2)) * p.ve.x_stride + 8 * (tid & 3));
  const auto rt = make_rsrc(p.ve.table, p.table_bytes);
  const int ch = tid % S::CPR;
  for (int base = 0; base < npair; base += S::U * S::PPP) {
    u32x4 dd[S::U], ee[S::U];
    int id[S::U];
    float g[S::U];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int i = min(base + u * S::PPP + tid / S::CPR, npair - 1);  // (duplicates are not stored)
      id[u] = p.ve.ids[r0 + i / H];
      g[u] = p.gate[rh0 + i];
      dd[u] = ld16((const bf16*)p.dv + (rh0 + i) * D + 8 * ch);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int i = min(base + u * S::PPP + tid / S::CPR, npair - 1);
      ee[u] = ve_chunk(rt, p.table_bytes, id[u], H, D, i % H, ch);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
      const int i = base + u * S::PPP + tid / S::CPR;
      float d[8], e[8];
      unpack8(dd[u], d);
      unpack8(ee[u], e);
      float dot = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        dot = __builtin_fmaf(d[k], e[k], dot);
        d[k] *= g[u];
      }
      dot = group_sum<S::CPR>(dot);
      if (i < npair) {
        st16((bf16*)p.dve + (rh0 + i) * D + 8 * ch, pack8(d));
        if (ch == 0) zs[i] = dot * g[u] * (1.f - 0.5f * g[u]);
      }
    }
  }
  if (tid < 4 * kVeRows) {
    float f[8];
    unpack8(xrow, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[tid >> 2][8 * (tid & 3) + e] = f[e];
  }
  for (int e = tid; e < H * 32; e += 256) wsh[e / 32][e % 32] = (float)((const bf16*)p.ve.w)[e];
  __syncthreads();
  for (int e = tid; e < nr * 32; e += 256) {
    const int r = e / 32, c = e % 32;
    float s = 0.f;
    for (int h = 0; h < H; ++h) s = __builtin_fmaf(zs[r * H + h], wsh[h][c], s);
    p.dx32[(r0 + r) * 32 + c] = s;
  }
  const int c = tid % 32, j = tid / 32;
  for (int h = 0; h < H; ++h) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kVeRows / 8; ++r) {
      const int rr = j + 8 * r;
      if (rr < nr) s = __builtin_fmaf(zs[rr * H + h], xs[rr][c], s);
    }
    acc[j][h][c] = s;
  }
  __syncthreads();
  for (int e = tid; e < H * 32; e += 256) {
    const int h = e / 32, cc = e % 32;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) s += acc[q][h][cc];
    p.part[(long)e * nblk + blockIdx.x] = s;
  }
}

// dw[e] (e = h * 32 + c) = the sum of the blocks' partials part[e * nblk ..]:
// one wave per e; lane l adds blocks l, l + 64, ... in order, then the lanes'
// sums are added by a fixed butterfly (fixed order: deterministic).
__global__ void __launch_bounds__(64) ve_bwd_reduce_kernel(VeBwdParams p, int nblk) {
  const int e = blockIdx.x, l = threadIdx.x;
  const float* src = p.part + (long)e * nblk;
  float s = 0.f;
  for (int k0 = l; k0 < nblk; k0 += 8 * 64) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = k0 + 64 * u < nblk ? src[k0 + 64 * u] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (l == 0) p.dw[e] = s;
}

hipError_t launch_ve_bwd(const VeBwdParams& p, int head_dim, hipStream_t stream) {
  const int nblk = (int)((p.rows + kVeRows - 1) / kVeRows);
  if (head_dim == 128)
    hipLaunchKernelGGL((ve_bwd_kernel<128>), dim3((unsigned)nblk), dim3(256), 0, stream, p, nblk);
  else
    hipLaunchKernelGGL((ve_bwd_kernel<64>), dim3((unsigned)nblk), dim3(256), 0, stream, p, nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ve_bwd_reduce_kernel, dim3((unsigned)(p.Hkv * 32)), dim3(64), 0, stream, p, nblk);
  return hipGetLastError();
}

}  // namespace sa
