// Standalone weightless RMS norm of head rows (the QK-norm of the layer, run
// on its own): y = x / sqrt(mean(x^2) + eps) per row of head_dim values,
// plus the per-row 1/sqrt(mean(x^2) + eps).
// Sources: [post] QK-norm passage; [guide] 8.2.1 (RMSNorm via F.rms_norm).
// HBM-bound: one 16-byte chunk per lane, D/8 lanes per row, the sum of
// squares reduced across the row's lanes with DPP row operations. With
// rotary tables (internal use: [B, T, H] head rows) each row is also turned
// by the angles of its position, pairs of dimensions i and i + D/2.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

template <int D>
__global__ void __launch_bounds__(256) qknorm_kernel(NormParams p) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int sub = threadIdx.x % CPR;
  for (long row = (long)blockIdx.x * RPB + threadIdx.x / CPR; row < p.rows; row += (long)gridDim.x * RPB) {
    float x[8];
    unpack8(ld16((const bf16*)p.x + row * D + 8 * sub), x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
    if (p.rope.cos != nullptr) {
      float xp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xp[e] = __shfl_xor(x[e], CPR / 2);
      const long t = (row / p.H) % p.T;
      const long tr = t * p.rope.stride + 8 * (sub % (CPR / 2));
      rope8(x, xp, p.rope.cos + tr, p.rope.sin + tr, sub >= CPR / 2, false);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= r;
    st16((bf16*)p.y + row * D + 8 * sub, pack8(x));
    if (p.rstd != nullptr && sub == 0) p.rstd[row] = r;
  }
}

hipError_t launch_qknorm(const NormParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev) {
  const int rpb = 256 / (head_dim / 8);
  const long nblk = (p.rows + rpb - 1) / rpb;
  const unsigned grid = (unsigned)(nblk < 16384L ? nblk : 16384L);
  if (head_dim == 128)
    hipExtLaunchKernelGGL((qknorm_kernel<128>), dim3(grid), dim3(256), 0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((qknorm_kernel<64>), dim3(grid), dim3(256), 0, stream, ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

}  // namespace sa
