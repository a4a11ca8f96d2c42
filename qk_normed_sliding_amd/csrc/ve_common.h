// Device helpers of the value-embedding gate ("autoresearch Administrator &
// Developer Guide", section 8.2.1), shared by the forward's key/value
// prologue and the backward's value-embedding passes.
#pragma once

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

// gate of row `row` (= b*T + t) and KV head h, from x[row][0..31] and w[h][0..31]
__device__ __forceinline__ float ve_gate_of(const VeParams& ve, long row, int h) {
  const bf16* xr = (const bf16*)ve.x + row * ve.x_stride;
  const bf16* wr = (const bf16*)ve.w + (long)h * 32;
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a[8], c[8];
    unpack8(ld16(xr + 8 * j), a);
    unpack8(ld16(wr + 8 * j), c);
#pragma unroll
    for (int e = 0; e < 8; ++e) z = __builtin_fmaf(a[e], c[e], z);
  }
  return 2.f / (1.f + __expf(-z));
}

// 16 bytes (8 elements) of the embedding row of `row`, head h, chunk ch; an
// id outside the table (table_bytes long) gives zeros. The offset is checked
// in 64 bits before it becomes the buffer load's 32-bit offset.
__device__ __forceinline__ u32x4 ve_chunk(const VeParams& ve, __amdgpu_buffer_rsrc_t rt, uint32_t table_bytes,
                                          long row, int Hkv, int D, int h, int ch) {
  const int id = ve.ids[row];
  const long off = ((long)id * Hkv * D + (long)h * D + 8 * ch) * 2;
  return (id < 0 || off >= (long)table_bytes) ? u32x4{0u, 0u, 0u, 0u} : bload16(rt, (uint32_t)off);
}

}  // namespace sa
