// Muon's polar-express orthogonalisation ("autoresearch Administrator &
// Developer Guide", section 8.2.3) for stacks of bf16 matrices: the gradient
// scaled by its Frobenius norm, then five steps
//   A = X X^T,  B = b A + c A A,  X <- a X + B X
// on the wide side (a tall matrix is turned into a wide one by a transpose
// on the way in and out: the iteration commutes with transposition).
//
// The contractions are batched bf16 GEMMs on the matrix cores with fp32
// accumulation, C = alpha A op(B) + beta C0, op(B) = B^T ("bt": B given as
// [N][K], both operands read along K) or B ("bn": B given as [K][N], read
// with LDS transpose reads). A 256-thread workgroup owns a 128 x 128 tile of
// C (a 64 x 64 quarter per wave, 2 x 2 blocks of 32 x 32); K advances in
// steps of 64 through two LDS stages filled by direct buffer-to-LDS copies,
// XOR-swizzled so that the operand reads are bank-conflict free. The MFMA
// takes the N-side operand first, so each lane's accumulators hold one row of
// C (16 columns) and the epilogue stores 8 bytes per (lane, register quad).
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

template <bool BN>
__global__ void __launch_bounds__(256) gemm_kernel(GemmParams p) {
  constexpr int TM = 128, TN = 128, TK = 64;
  __shared__ __attribute__((aligned(1024))) bf16 As[2][TM * TK];  // [m][k], 8 chunks per row
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][TN * TK];  // bt: [n][k] (8 chunks); bn: [k][n] (16 chunks)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;  // this wave's 64 x 64 quarter of the tile
  const int tiles_n = p.N / TN;
  const int m0 = (blockIdx.x / tiles_n) * TM;
  const int n0 = (blockIdx.x % tiles_n) * TN;
  const long bz = blockIdx.y;

  const bf16* A = (const bf16*)p.a + bz * p.M * p.K;
  const bf16* B = (const bf16*)p.b + bz * p.N * p.K;
  const u32x4 ra = rsrc_words(A, (uint32_t)(p.M * p.K * 2));
  const u32x4 rb = rsrc_words(B, (uint32_t)(p.N * p.K * 2));

  // Copies: instruction j of wave w fills the 1 KB block blk = 4j + w of a
  // tile. [x][k] tiles (8 chunks per row): rows 8 blk + lane/8; the row's
  // swizzle depends on blk only through its parity, which is w's. [k][n]
  // tiles (16 chunks per row): rows 4 blk + lane/16; swizzle from blk mod 4 = w.
  uint32_t oa, ob;
  {
    const int r8 = (w & 1) * 8 + lane / 8;
    oa = (uint32_t)((lane / 8) * p.K + 8 * ((lane % 8) ^ swz<8>(r8))) * 2;
    if constexpr (BN) {
      const int r16 = (w & 3) * 4 + lane / 16;
      ob = (uint32_t)((lane / 16) * p.N + 8 * ((lane % 16) ^ swz<16>(r16))) * 2;
    } else {
      ob = oa;
    }
  }
  auto issue = [&](int ks, int st) {
    const int k0 = ks * TK;
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * j + w;
      dma16(ra, uniform((int)(la + blk * 1024)), oa + (uint32_t)(((m0 + 8 * blk) * p.K + k0) * 2), 0u);
      if constexpr (BN)
        dma16(rb, uniform((int)(lb + blk * 1024)), ob + (uint32_t)(((k0 + 4 * blk) * p.N + n0) * 2), 0u);
      else
        dma16(rb, uniform((int)(lb + blk * 1024)), ob + (uint32_t)(((n0 + 8 * blk) * p.K + k0) * 2), 0u);
    }
  };

  // Operand reads. Row reads ([x][k] tiles): row 32 blk + l32, k = 16 kk +
  // 8 half + e in chunk 2kk + half. Transpose reads ([k][n] tile): rows 16 kk
  // + 8 half + tq (+4), columns 32 blk + 16 g1 + 4 qq; lane l receives
  // column 32 blk + l32 at k = 16 kk + 8 half + e, the same K order.
  auto row_op = [&](uint32_t base, int blk, int kk) {
    const int r = 32 * blk + l32;
    return *(SA_LDS const bf16x8*)(uintptr_t)(base + (uint32_t)(r * 128 + (((2 * kk + half) ^ swz<8>(r)) << 4)));
  };
  uint32_t trb[2] = {0u, 0u};
  if constexpr (BN) {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) trb[hi] = (uint32_t)swz_off<16>(8 * half + tq + 4 * hi, 16 * g1 + 4 * qq) * 2;
  }
  auto tr_op = [&](uint32_t base, int blk, int kk) {
    const uint32_t rbase = base + (uint32_t)(kk * 16 * 256);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (SA_LDS bf16x4*)(uintptr_t)(rbase + (trb[0] ^ (uint32_t)(blk << 6))));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (SA_LDS bf16x4*)(uintptr_t)(rbase + (trb[1] ^ (uint32_t)(blk << 6))));
    return cat(lo, hi);
  };

  f32x16 acc[2][2];  // [n block][m block]: register 4i + j of lane l = C[row l32][column 8i + 4half + j]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int nk = p.K / TK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < nk) issue(ks + 1, st ^ 1);  // the other stage was last read before the previous barrier
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
    bf16x8 bo[4][2], ao[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        bo[kk][x] = row_op(la, 2 * wm + x, kk);
        if constexpr (BN)
          ao[kk][x] = tr_op(lb, 2 * wn + x, kk);
        else
          ao[kk][x] = row_op(lb, 2 * wn + x, kk);
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = mfma32(ao[kk][x], bo[kk][y], acc[x][y]);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next stage have landed
    __syncthreads();
  }

  // epilogue: C = alpha acc + beta C0 (bf16)
  const long cbase = bz * p.M * p.N;
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const long row = m0 + 32 * (2 * wm + y) + l32;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long off = cbase + row * p.N + n0 + 32 * (2 * wn + x) + 8 * i + 4 * half;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = p.alpha * acc[x][y][4 * i + j];
        if (p.c0 != nullptr) {
          const u32x2 c0 = *(const u32x2*)((const bf16*)p.c0 + off);
          v[0] += p.beta * __uint_as_float(c0[0] << 16);
          v[1] += p.beta * __uint_as_float(c0[0] & 0xffff0000u);
          v[2] += p.beta * __uint_as_float(c0[1] << 16);
          v[3] += p.beta * __uint_as_float(c0[1] & 0xffff0000u);
        }
        u32x2 o;
        o[0] = pack2(v[0], v[1]);
        o[1] = pack2(v[2], v[3]);
        *(u32x2*)((bf16*)p.c + off) = o;
      }
  }
}

// Sum of squares of chunk blockIdx.x of matrix blockIdx.y (elements
// [chunk * per, (chunk + 1) * per)), in a fixed order: part[y * gridDim.x + x].
__global__ void __launch_bounds__(256) sumsq_kernel(const bf16* x, float* part, long per_matrix, long per) {
  __shared__ float red[4];
  const bf16* base = x + (long)blockIdx.y * per_matrix + (long)blockIdx.x * per;
  float s = 0.f;
  for (long e = 8L * threadIdx.x; e < per; e += 8L * 256) {
    float f[8];
    unpack8(ld16(base + e), f);
#pragma unroll
    for (int k = 0; k < 8; ++k) s += f[k] * f[k];
  }
  // wave sum: groups of 16 (DPP), then across the four rows of the wave
  s = group_sum<16>(s);
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[(long)blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// y = x / (sqrt(sum of the matrix's partial sums) + eps), chunk blockIdx.x of matrix blockIdx.y.
__global__ void __launch_bounds__(256) scale_kernel(const bf16* x, bf16* y, const float* part, long per_matrix,
                                                    long per, float eps) {
  const float* pm = part + (long)blockIdx.y * gridDim.x;
  float ss = 0.f;
  for (int c = 0; c < (int)gridDim.x; ++c) ss += pm[c];  // same order in every workgroup
  const float sc = 1.f / (sqrtf(ss) + eps);
  const long off = (long)blockIdx.y * per_matrix + (long)blockIdx.x * per;
  for (long e = 8L * threadIdx.x; e < per; e += 8L * 256) {
    float f[8];
    unpack8(ld16(x + off + e), f);
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] *= sc;
    st16(y + off + e, pack8(f));
  }
}

// out[b][c][r] = in[b][r][c] for 64 x 64 tiles (R, C multiples of 64).
__global__ void __launch_bounds__(256) transpose_kernel(const bf16* in, bf16* out, int R, int C) {
  __shared__ unsigned short t[64][66];
  const int tr = blockIdx.x / (C / 64), tc = blockIdx.x % (C / 64);
  const long mb = (long)blockIdx.y * R * C;
  const unsigned short* src = (const unsigned short*)in + mb;
  unsigned short* dst = (unsigned short*)out + mb;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;
    t[r][c] = src[(long)(64 * tr + r) * C + 64 * tc + c];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int c = e / 64, r = e % 64;
    dst[(long)(64 * tc + c) * R + 64 * tr + r] = t[r][c];
  }
}

hipError_t launch_gemm(const GemmParams& p, bool b_kn, int batch, hipStream_t stream) {
  const dim3 grid((unsigned)((p.M / 128) * (p.N / 128)), (unsigned)batch);
  if (b_kn)
    hipLaunchKernelGGL((gemm_kernel<true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fro_scale(const void* x, void* y, float* part, int batch, long per_matrix, float eps,
                            hipStream_t stream) {
  const long per = per_matrix / kFroChunks;
  const dim3 grid((unsigned)kFroChunks, (unsigned)batch);
  hipLaunchKernelGGL(sumsq_kernel, grid, dim3(256), 0, stream, (const bf16*)x, part, per_matrix, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scale_kernel, grid, dim3(256), 0, stream, (const bf16*)x, (bf16*)y, (const float*)part,
                     per_matrix, per, eps);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* in, void* out, int batch, int R, int C, hipStream_t stream) {
  const dim3 grid((unsigned)((R / 64) * (C / 64)), (unsigned)batch);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, (const bf16*)in, (bf16*)out, R, C);
  return hipGetLastError();
}

}  // namespace sa
