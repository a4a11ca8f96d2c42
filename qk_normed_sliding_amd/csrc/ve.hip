// Value-embedding gate of the value rows ("autoresearch Administrator &
// Developer Guide", section 8.2.1: alternating layers, the last always, mix a
// learned embedding of the token ids into v):
//   g[b,t,h] = 2 sigmoid(sum_c x[b,t,c] w[h,c]), c < 32,
//   v'[b,t,h,:] = v[b,t,h,:] + g[b,t,h] ve[b,t,h,:],  ve = table[ids[b,t]] viewed [Hkv, D].
// The forward writes v' and g once (ve_prep_kernel) into its workspace and
// runs the attention on v'; the backward reads them back from there (or
// writes them itself without the forward's workspace), runs its kernels on
// v', then maps dL/dv' to the embedding, gate and input gradients:
//   dve = g dv',  dz = <dv', ve> g (1 - g/2),  dx32 = dz w,  dw = sum_{b,t} dz^T x32,
// the last as fixed-order partial sums per block of rows and one reduction.
// dv (the raw v's gradient) is dv' itself. Embedding rows are read through a
// buffer descriptor over the table: an id past the table reads zeros.
#include "sa_common.h"
#include "sa_kernels.h"
#include "ve_common.h"

namespace sa {

// v' and g for the backward: one 16-byte chunk per lane, D/8 lanes per (row, head).
template <int D>
__global__ void __launch_bounds__(256) ve_prep_kernel(VePrepParams p) {
  constexpr int CPR = D / 8;
  const long nrh = (long)p.rows * p.Hkv;
  const auto rt = make_rsrc(p.ve.table, p.table_bytes);
  const int ch = threadIdx.x % CPR;
  for (long rh = (long)blockIdx.x * (256 / CPR) + threadIdx.x / CPR; rh < nrh; rh += (long)gridDim.x * (256 / CPR)) {
    const long row = rh / p.Hkv;
    const int h = (int)(rh % p.Hkv);
    const float g = ve_gate_of(p.ve, row, h);
    float v[8], e[8];
    unpack8(ld16((const bf16*)p.v + rh * D + 8 * ch), v);
    unpack8(ve_chunk(p.ve, rt, p.table_bytes, row, p.Hkv, D, h, ch), e);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(g, e[k], v[k]);
    st16((bf16*)p.v_mixed + rh * D + 8 * ch, pack8(v));
    if (ch == 0) p.gate[rh] = g;
  }
}

// dve = g dv' and dz = <dv', ve> g (1 - g/2) per (row, head): D/8 lanes per
// (row, head), the dot reduced over those lanes.
template <int D>
__global__ void __launch_bounds__(256) ve_bwd_rows_kernel(VeBwdParams p) {
  constexpr int CPR = D / 8;
  const long nrh = (long)p.rows * p.Hkv;
  const auto rt = make_rsrc(p.ve.table, p.table_bytes);
  const int ch = threadIdx.x % CPR;
  for (long rh = (long)blockIdx.x * (256 / CPR) + threadIdx.x / CPR; rh < nrh; rh += (long)gridDim.x * (256 / CPR)) {
    const long row = rh / p.Hkv;
    const int h = (int)(rh % p.Hkv);
    const float g = p.gate[rh];
    float d[8], e[8];
    unpack8(ld16((const bf16*)p.dv + rh * D + 8 * ch), d);
    unpack8(ve_chunk(p.ve, rt, p.table_bytes, row, p.Hkv, D, h, ch), e);
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      dot = __builtin_fmaf(d[k], e[k], dot);
      d[k] *= g;
    }
    st16((bf16*)p.dve + rh * D + 8 * ch, pack8(d));
    dot = group_sum<CPR>(dot);
    if (ch == 0) p.dz[rh] = dot * g * (1.f - 0.5f * g);
  }
}

// Per block of kVeRows rows: dx32[row][c] = sum_h dz[row][h] w[h][c], and the
// block's partial dw[h][c] = sum_row dz[row][h] x[row][c]. The block's x rows
// (16-byte loads), dz and w are staged in LDS first. For dw, thread (j, c)
// sums rows j, j + 8, ... of the block for every head; the 8 row groups are
// then added in order (fixed order: deterministic).
__global__ void __launch_bounds__(256) ve_bwd_gate_kernel(VeBwdParams p) {
  static_assert(kVeRows == 64, "one 16-byte chunk of x per thread");
  __shared__ float xs[kVeRows][33];
  __shared__ float zs[kVeRows][kVeMaxHeads + 1];
  __shared__ float wsh[kVeMaxHeads][32];
  __shared__ float acc[8][kVeMaxHeads][32];
  const int tid = threadIdx.x;
  const long r0 = (long)blockIdx.x * kVeRows;
  const int nr = (int)min((long)kVeRows, p.rows - r0);
  const int H = p.Hkv;
  {
    const int r = tid >> 2, ch = tid & 3;
    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < nr) unpack8(ld16((const bf16*)p.ve.x + (r0 + r) * p.ve.x_stride + 8 * ch), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[r][8 * ch + e] = f[e];
  }
  for (int e = tid; e < nr * H; e += 256) zs[e / H][e % H] = p.dz[r0 * H + e];
  for (int e = tid; e < H * 32; e += 256) wsh[e / 32][e % 32] = (float)((const bf16*)p.ve.w)[e];
  __syncthreads();
  for (int e = tid; e < nr * 32; e += 256) {
    const int r = e / 32, c = e % 32;
    float s = 0.f;
    for (int h = 0; h < H; ++h) s = __builtin_fmaf(zs[r][h], wsh[h][c], s);
    p.dx32[(r0 + r) * 32 + c] = s;
  }
  const int c = tid % 32, j = tid / 32;
  for (int h = 0; h < H; ++h) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kVeRows / 8; ++r) {
      const int rr = j + 8 * r;
      if (rr < nr) s = __builtin_fmaf(zs[rr][h], xs[rr][c], s);
    }
    acc[j][h][c] = s;
  }
  __syncthreads();
  for (int e = tid; e < H * 32; e += 256) {
    const int h = e / 32, cc = e % 32;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) s += acc[g][h][cc];
    p.part[(long)blockIdx.x * H * 32 + e] = s;
  }
}

// dw[h][c] = sum of the blocks' partials: workgroup (h, column group cg of 8
// columns), thread (j, c) sums blocks j, j + 32, ... (loads in groups of 8),
// and the 32 sums are added in order (fixed order: deterministic).
__global__ void __launch_bounds__(256) ve_bwd_reduce_kernel(VeBwdParams p, int nblk) {
  __shared__ float acc[32][8];
  const int h = blockIdx.x / 4, cg = blockIdx.x % 4;
  const int c = threadIdx.x % 8, j = threadIdx.x / 8;
  const int col = 8 * cg + c;
  float s = 0.f;
  for (int k0 = j; k0 < nblk; k0 += 256) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 32 * u;
      t[u] = k < nblk ? p.part[((long)k * p.Hkv + h) * 32 + col] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += t[u];
  }
  acc[j][c] = s;
  __syncthreads();
  if (j == 0) {
    float r = 0.f;
#pragma unroll
    for (int g = 0; g < 32; ++g) r += acc[g][c];
    p.dw[h * 32 + col] = r;
  }
}

hipError_t launch_ve_prep(const VePrepParams& p, int head_dim, hipStream_t stream) {
  const long nrh = (long)p.rows * p.Hkv;
  const long per = 256 / (head_dim / 8);
  const unsigned grid = (unsigned)min((nrh + per - 1) / per, 16384L);
  if (head_dim == 128)
    hipLaunchKernelGGL((ve_prep_kernel<128>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((ve_prep_kernel<64>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_ve_bwd(const VeBwdParams& p, int head_dim, hipStream_t stream) {
  const long nrh = (long)p.rows * p.Hkv;
  const long per = 256 / (head_dim / 8);
  const unsigned grid = (unsigned)min((nrh + per - 1) / per, 16384L);
  if (head_dim == 128)
    hipLaunchKernelGGL((ve_bwd_rows_kernel<128>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((ve_bwd_rows_kernel<64>), dim3(grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nblk = (int)((p.rows + kVeRows - 1) / kVeRows);
  hipLaunchKernelGGL(ve_bwd_gate_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ve_bwd_reduce_kernel, dim3((unsigned)(p.Hkv * 4)), dim3(256), 0, stream, p, nblk);
  return hipGetLastError();
}

}  // namespace sa
