// Standalone weightless RMS norm of head rows (the QK-norm of the layer, run
// on its own): y = x / sqrt(mean(x^2) + eps) per row of head_dim values,
// plus the per-row 1/sqrt(mean(x^2) + eps).
// Sources: [post] QK-norm passage; [guide] 8.2.1 (RMSNorm via F.rms_norm).
// HBM-bound: one 16-byte chunk per lane, D/8 lanes per row, the sum of
// squares reduced across the row's lanes with DPP row operations. With
// rotary tables (internal use: [B, T, H] head rows) each row is also turned
// by the angles of its position, pairs of dimensions i and i + D/2. The
// forward's (and the recomputing backward's) pass over the k rows also writes
// the value-embedding mix v' and its gate when the layer has one.
#include "sa_common.h"
#include "sa_kernels.h"
#include "ve_common.h"

namespace sa {

// VE: the same launch also mixes the value rows (value-embedding gate): its
// first nv_blocks workgroups write v' and g, one (row, head) pair per D/8
// lanes, and the rest norm the rows.
template <int D, bool VE>
__global__ void __launch_bounds__(256) qknorm_kernel(NormParams p, VePrepParams pv, int nv_blocks) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const int sub = threadIdx.x % CPR;
  long first = blockIdx.x, stride = gridDim.x;
  if constexpr (VE) {
    if ((int)blockIdx.x < nv_blocks) {
      const long rh = (long)blockIdx.x * RPB + threadIdx.x / CPR;
      if (rh < pv.rows * pv.Hkv) ve_prep_pair<D>(pv, make_rsrc(pv.ve.table, pv.table_bytes), rh, sub);
      return;
    }
    first -= nv_blocks;
    stride -= nv_blocks;
  }
  for (long row = first * RPB + threadIdx.x / CPR; row < p.rows; row += stride * RPB) {
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

hipError_t launch_qknorm(const NormParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev,
                         const VePrepParams* ve) {
  const int rpb = 256 / (head_dim / 8);
  const long nblk = (p.rows + rpb - 1) / rpb;
  const int nk = (int)(nblk < 16384L ? nblk : 16384L);
  const int nv = ve ? (int)((ve->rows * ve->Hkv + rpb - 1) / rpb) : 0;
  const VePrepParams pv = ve ? *ve : VePrepParams{};
  const dim3 grid((unsigned)(nv + nk));
  if (head_dim == 128) {
    if (ve)
      hipExtLaunchKernelGGL((qknorm_kernel<128, true>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p, pv, nv);
    else
      hipExtLaunchKernelGGL((qknorm_kernel<128, false>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p, pv, 0);
  } else {
    if (ve)
      hipExtLaunchKernelGGL((qknorm_kernel<64, true>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p, pv, nv);
    else
      hipExtLaunchKernelGGL((qknorm_kernel<64, false>), grid, dim3(256), 0, stream, ev.start, ev.stop, 0, p, pv, 0);
  }
  return hipGetLastError();
}

}  // namespace sa
