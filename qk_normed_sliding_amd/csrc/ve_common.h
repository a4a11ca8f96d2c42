// Device helpers of the value-embedding gate ("autoresearch Administrator &
// Developer Guide", section 8.2.1: g = 2 sigmoid(x[:32] w_h), v' = v + g ve),
// shared by the forward's norm pass (which also writes v' and g) and the
// backward's gate passes.
#pragma once

#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

// 16 bytes (8 elements) of the embedding row of token `id`, head h, chunk ch;
// an id outside the table (table_bytes long) reads zeros: the offset is
// checked in 64 bits and replaced by one past the buffer's range, so the load
// itself is unconditional.
__device__ __forceinline__ u32x4 ve_chunk(__amdgpu_buffer_rsrc_t rt, uint32_t table_bytes, int id, int Hkv, int D,
                                          int h, int ch) {
  const long off = ((long)id * Hkv * D + (long)h * D + 8 * ch) * 2;
  return bload16(rt, (id < 0 || off >= (long)table_bytes) ? table_bytes : (uint32_t)off);
}

// The gate's input channels that lane ch of a (row, head) group of CPR lanes
// takes: (32/CPR)ch .. of x's row and of w's row h, as packed bf16 pairs.
template <int CPR>
struct VeGateIn {
  static constexpr int XPL = 32 / CPR;
  static_assert(XPL == 2 || XPL == 4, "16 or 8 lanes per row and head");
  uint32_t x[XPL / 2], w[XPL / 2];
  __device__ __forceinline__ void load(const VeParams& ve, long row, int h, int ch) {
    const uint32_t* xr = (const uint32_t*)((const bf16*)ve.x + row * ve.x_stride + XPL * ch);
    const uint32_t* wr = (const uint32_t*)((const bf16*)ve.w + (long)h * 32 + XPL * ch);
#pragma unroll
    for (int i = 0; i < XPL / 2; ++i) {
      x[i] = xr[i];
      w[i] = wr[i];
    }
  }
  // g = 2 sigmoid(<x, w>), the products summed over the group's lanes (every lane gets g)
  __device__ __forceinline__ float gate() const {
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < XPL / 2; ++i) {
      z = __builtin_fmaf(__uint_as_float(x[i] << 16), __uint_as_float(w[i] << 16), z);
      z = __builtin_fmaf(__uint_as_float(x[i] & 0xffff0000u), __uint_as_float(w[i] & 0xffff0000u), z);
    }
    z = group_sum<CPR>(z);
    return 2.f / (1.f + __expf(-z));
  }
};

// v' = v + g ve and g for pair rh = row * Hkv + h, chunk ch of D/8 (the pair's
// D/8 lanes run this together: the gate's dot product is summed over them).
template <int D>
__device__ __forceinline__ void ve_prep_pair(const VePrepParams& p, __amdgpu_buffer_rsrc_t rt, long rh, int ch) {
  const long row = rh / p.Hkv;
  const int h = (int)(rh % p.Hkv);
  const int id = p.ve.ids[row];
  VeGateIn<D / 8> gi;
  gi.load(p.ve, row, h, ch);
  const u32x4 vv = ld16((const bf16*)p.v + rh * D + 8 * ch);
  const u32x4 ee = ve_chunk(rt, p.table_bytes, id, p.Hkv, D, h, ch);
  const float g = gi.gate();
  float v[8], e[8];
  unpack8(vv, v);
  unpack8(ee, e);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = __builtin_fmaf(g, e[k], v[k]);
  st16((bf16*)p.v_mixed + rh * D + 8 * ch, pack8(v));
  if (ch == 0) p.gate[rh] = g;
}

}  // namespace sa
