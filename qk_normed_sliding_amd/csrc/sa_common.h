// Shared device helpers for the gfx950 (CDNA4) attention kernels.
//
// Register-layout facts the kernels rely on (64-lane wavefronts):
//   v_mfma_f32_32x32x16_bf16: A is 32(M)x16(K), B is 16(K)x32(N); lane l holds
//   8 consecutive-K operands of row/col l%32 in K-half l/32 (the same K
//   assignment for A and B, so any consistent relabelling of K is a valid
//   contraction). Accumulator register r = 4i + j of lane l holds
//   C[8i + 4(l/32) + j][l%32].
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
//   (i%4) of the 4 x bf16 read by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
//   Reading row-major B[k][n] with lane 4t+q addressing &B[k0+t][n0+4q] hands
//   lane i the column B[k0..k0+3][n0+i]: a K-major MFMA operand straight
//   from a row-major LDS tile, with no transposed copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define SA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 4 x bf16 transposed LDS read (see the header comment for the lane mapping).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// Sum / max over the lane pair (l, l^32).
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over aligned groups of 8 or 16 consecutive lanes (DPP row operations).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp<0xB1>(x);                         // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                         // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Raw buffer loads: a scalar resource (base, byte range) plus a 32-bit lane
// offset. Reads at or past `bytes` return zero, which zero-fills ragged tails
// without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// As bload16 with the non-temporal (streaming) cache policy: for rows read once,
// so that they do not displace data the L2 cache serves again.
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
// Raw buffer store: writes at or past the resource's byte range are dropped,
// so a store of a ragged tail needs no branch (and is always issued).
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}
// As bstore16 with the non-temporal (streaming) cache policy: for whole-row results
// that nothing in the same pass reads again, so they do not displace the tiles
// that the L2 cache still serves.
__device__ __forceinline__ void bstore16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 2);
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_off, 0, 0);
}

// Buffer resource as four dwords (base address, stride 0, size in bytes,
// flags), uniform across the wave so that it lives in scalar registers.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from a buffer straight into LDS: lane l fills bytes
// [16l, 16l+16) after lds_base (a wave-uniform LDS byte address); offsets
// past the buffer's size read as zero. Issued from inline assembly so that
// the compiler does not count it as a pending LDS write (it would otherwise
// wait for it before every later LDS read and barrier): the issuing wave
// waits for it itself (vmcnt) before the barrier that publishes the data.
// The byte offset is voff (per lane) + soff (wave-uniform); the range check
// against the buffer's size applies to voff alone.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");  // m0 is reserved by the compiler, which reloads it before each of its own uses
}
// As dma16 with 4 bytes per lane: lane l fills bytes [4l, 4l+4) after lds_base.
__device__ __forceinline__ void dma4(u32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(SA_LDS const void*)p;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }

__device__ __forceinline__ void unpack8(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Rotary embedding of 8 values x[e] of one row, dimensions i0 + e of the
// lower half (upper = false) or i0 + D/2 + e of the upper half, given the
// values xp[e] of the other half's partner dimensions and the table rows
// c = cos + i0, s = sin + i0 (16-byte aligned): the pair (a, b) = (lower,
// upper) turns to (a c - b s, a s + b c). With back = true the transposed
// (inverse) turn: (a c + b s, -a s + b c).
__device__ __forceinline__ void rope8(float* x, const float* xp, const float* c, const float* s, bool upper,
                                      bool back) {
  const f32x4 c0 = *(const f32x4*)c, c1 = *(const f32x4*)(c + 4);
  const f32x4 s0 = *(const f32x4*)s, s1 = *(const f32x4*)(s + 4);
  // lower: x c - xp s (back: x c + xp s); upper: x c + xp s (back: x c - xp s)
  const float sg = (upper != back) ? 1.f : -1.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ce = e < 4 ? c0[e] : c1[e - 4];
    const float se = e < 4 ? s0[e] : s1[e - 4];
    x[e] = __builtin_fmaf(x[e], ce, sg * xp[e] * se);
  }
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 r;
  r[0] = (bf16)a;
  r[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack2(f[2 * i], f[2 * i + 1]);
  return w;
}

// Swap bits 2 and 3 of a 5-bit row index. Reading MFMA A-operand rows in this
// order makes accumulator registers 8s..8s+7 of a lane hold 8 consecutive
// rows (16s + 8(l/32) + 0..7), which is exactly the K-slot order of the next
// MFMA's operand, so P and dS feed the next contraction without a shuffle.
__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Swizzle of 16-byte chunks in LDS rows without padding: chunk j of row r is
// stored at chunk j ^ f(r). For rows of 16 chunks f(r) puts the low two row
// bits on the high chunk bits and vice versa; for rows of 8 chunks it uses
// row bits 1..3. Both make 16 consecutive rows read at one logical chunk, and
// 4 consecutive rows read at 4 consecutive chunks, land on distinct banks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}
template <int CH>
__device__ __forceinline__ int swz_off(int r, int col) {  // element offset of (row, col)
  return r * CH * 8 + ((((col >> 3) ^ swz<CH>(r)) & (CH - 1)) << 3) + (col & 7);
}

}  // namespace sa
