// Muon's polar-express orthogonalisation ("autoresearch Administrator &
// Developer Guide", section 8.2.3) for stacks of bf16 matrices: the gradient
// scaled by its Frobenius norm, then five steps
//   A = X X^T,  B = b A + c A A,  X <- a X + B X
// on the wide side; a tall matrix Y is iterated as it is, as the transpose
// of the wide iterate (A = Y^T Y, Y <- Y B + a Y with B symmetric).
//
// The contractions are batched bf16 GEMMs on the matrix cores with fp32
// accumulation, C = alpha A op(B) + beta C0, op(B) = B^T ("bt": B given as
// [N][K], both operands read along K) or B ("bn": B given as [K][N], read
// with LDS transpose reads). A 256-thread workgroup owns a 128 x 128 tile of
// C (a 64 x 64 quarter per wave, 2 x 2 blocks of 32 x 32), a 64 x 64 tile
// (bt only; a 32 x 32 block per wave, up to four workgroups per compute
// unit, for products with few tiles), or (bn only) a
// 96 x 128 tile (a 96 x 32 column strip per wave, 3 blocks), which the host
// picks when its tile count fills the compute units' workgroup slots in
// fewer rounds of work (at m = 768: 1536 tiles, three full rounds of 512,
// against 1152 tiles of 128 x 128 in two and a quarter); K advances in
// steps of 64 through two LDS stages filled by direct buffer-to-LDS copies,
// XOR-swizzled so that the operand reads are bank-conflict free. The MFMA
// takes the N-side operand first, so each lane's accumulators hold one row of
// C (16 columns) and the epilogue stores 8 bytes per (lane, register quad).
// A symmetric product (X X^T, and A A with A symmetric) computes only the
// tiles on and above the diagonal and stores each off-diagonal tile mirrored
// as well. A product with few tiles and a long K splits K into equal ranges:
// each workgroup writes its fp32 partial tile and a second kernel adds the
// partials in a fixed order, applies alpha and beta and stores C (mirrored
// too when symmetric).
// The scaling by s = 1 / (||G||_F + eps) is folded into the first step: its
// Gram product is G G^T itself, whose diagonal sums to ||G||_F^2 (the
// product writes fixed-order partial sums of its diagonal blocks), and the
// next two products scale their alpha and beta by the powers of s that the
// scaled iteration implies (A A: c s^4 and b s^2; B X + a X: s and a s).
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

// Tile (tm, tn) of computed tile t: row-major over all tiles, or over the
// tiles with tm <= tn of a symmetric product.
__device__ __forceinline__ void tile_of(int t, int tiles_n, int sym, int& tm, int& tn) {
  if (sym) {
    tm = 0;
    while (t >= tiles_n - tm) {
      t -= tiles_n - tm;
      ++tm;
    }
    tn = tm + t;
  } else {
    tm = t / tiles_n;
    tn = t % tiles_n;
  }
}

// Work item of the workgroup with linear id L out of n, dealt round-robin to
// 8 XCDs: XCD x = L % 8 runs items [start(x), start(x + 1)) in order.
__device__ __forceinline__ int xcd_item(int L, int n) {
  constexpr int kXcds = 8;
  const int x = L % kXcds, slot = L / kXcds;
  const int per = n / kXcds, rem = n % kXcds;
  const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + slot;
}

// alpha and beta of a product, times s^npow_a and s^npow_b when the
// operand's scaling s = 1 / (||G||_F + eps) is folded in (the partial sums
// of ||G||_F^2 added in the same fixed order everywhere)
__device__ __forceinline__ void gemm_scales(const GemmParams& p, long bz, float& al, float& be) {
  al = p.alpha;
  be = p.beta;
  if (p.nsum != nullptr) {
    const float* pm = p.nsum + bz * p.nsum_n;
    float ss = 0.f;
    for (int c = 0; c < p.nsum_n; ++c) ss += pm[c];
    const float sc = 1.f / (sqrtf(ss) + p.neps);
    float fa = 1.f, fb = 1.f;
    for (int i = 0; i < p.npow_a; ++i) fa *= sc;
    for (int i = 0; i < p.npow_b; ++i) fb *= sc;
    al *= fa;
    be *= fb;
  }
}

// Epilogue of 32-row block y of a wave's part of C: C = alpha acc + beta C0
// (bf16) over NB column blocks of 32 (column col0 + 32 x + 8 i .. + 3 from
// register quad i of acc[x][y]). All of the block's C0 values are loaded
// before its first store: one memory round trip per block of rows rather
// than one per value (the stores could alias C0 as far as the compiler
// knows, so it would not move later loads above them). An off-diagonal tile
// of a symmetric product also goes to its mirror position, where 32 lanes
// store 32 consecutive elements of a row per instruction.
template <int NB, int MB>
__device__ __forceinline__ void gemm_store_rows(const GemmParams& p, long cbase, long row, long col0,
                                                const f32x16 (&acc)[NB][MB], int y, float al, float be,
                                                bool mirror) {
  u32x2 c0v[NB][4];
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) c0v[x][i] = u32x2{0u, 0u};
  if (p.c0 != nullptr) {
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c0v[x][i] = *(const u32x2*)((const bf16*)p.c0 + cbase + row * p.N + col0 + 32 * x + 8 * i);
  }
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long col = col0 + 32 * x + 8 * i;
      const u32x2 c0 = c0v[x][i];
      float v[4];
      v[0] = al * acc[x][y][4 * i + 0] + be * __uint_as_float(c0[0] << 16);
      v[1] = al * acc[x][y][4 * i + 1] + be * __uint_as_float(c0[0] & 0xffff0000u);
      v[2] = al * acc[x][y][4 * i + 2] + be * __uint_as_float(c0[1] << 16);
      v[3] = al * acc[x][y][4 * i + 3] + be * __uint_as_float(c0[1] & 0xffff0000u);
      u32x2 o;
      o[0] = pack2(v[0], v[1]);
      o[1] = pack2(v[2], v[3]);
      *(u32x2*)((bf16*)p.c + cbase + row * p.N + col) = o;
      if (mirror) {
        unsigned short* mc = (unsigned short*)p.c + cbase + col * p.M + row;
        mc[0] = (unsigned short)(o[0] & 0xffffu);
        mc[p.M] = (unsigned short)(o[0] >> 16);
        mc[2L * p.M] = (unsigned short)(o[1] & 0xffffu);
        mc[3L * p.M] = (unsigned short)(o[1] >> 16);
      }
    }
}

// AN: A given as [K][M] too (copied and read like B given as [K][N]), for
// the Gram product of a tall matrix Y, Y^T Y.
template <bool BN, int TM, bool AN = false>
__global__ void __launch_bounds__(256) gemm_kernel(GemmParams p) {
  constexpr int TN = TM == 64 ? 64 : 128, TK = 64;
  static_assert(TM == 128 || (TM == 96 && BN) || (TM == 64 && !BN),
                "128 x 128 tiles, 96 x 128 with B given as [K][N], or 64 x 64 with B given as [N][K]");
  static_assert(!AN || (BN && TM == 128), "A given as [K][M] with B given as [K][N] and 128 x 128 tiles");
  constexpr int MB = TM == 96 ? 3 : TM / 64;  // 32-row blocks per wave
  constexpr int NB = TM == 96 ? 1 : TM / 64;  // 32-column blocks per wave
  __shared__ __attribute__((aligned(1024))) bf16 As[2][TM * TK];  // [m][k], 8 chunks per row (an: [k][m], 16 chunks)
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][TN * TK];  // bt: [n][k] (8 chunks); bn: [k][n] (16 chunks)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // this wave's part of the tile: row blocks MB wm .., column blocks NB wn ..
  const int wm = TM == 96 ? 0 : w >> 1, wn = TM == 96 ? w : w & 1;
  const int tiles_n = p.N / TN;
  const int splits = p.splits > 1 ? p.splits : 1;
  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
  // work item w = (matrix, tile, split) in that order goes to the XCD that
  // runs a contiguous range of items, so the tiles of a matrix, which share
  // its row and column panels, meet in one L2.
  const int per_mat = gemm_tiles(p.M, p.N, p.sym, TM, TN) * splits;
  const int w_item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int tile = (w_item % per_mat) / splits, sp = w_item % splits;
  int tm, tn;
  tile_of(tile, tiles_n, p.sym, tm, tn);
  const int m0 = tm * TM;
  const int n0 = tn * TN;
  const long bz = w_item / per_mat;
  const int kbeg = sp * (p.K / splits);  // this workgroup's range of K

  const bf16* A = (const bf16*)p.a + bz * p.M * p.K;
  const bf16* B = (const bf16*)p.b + bz * p.N * p.K;
  const u32x4 ra = rsrc_words(A, (uint32_t)(p.M * p.K * 2));
  const u32x4 rb = rsrc_words(B, (uint32_t)(p.N * p.K * 2));

  // Copies: instruction j of wave w fills the 1 KB block blk = 4j + w of a
  // tile (A: TM / 8 blocks, B: TN / 8). [x][k] tiles (8 chunks per row): rows 8 blk + lane/8; the row's
  // swizzle depends on blk only through its parity, which is w's. [k][n]
  // tiles (16 chunks per row): rows 4 blk + lane/16; swizzle from blk mod 4 = w.
  uint32_t oa, ob;
  {
    const int r8 = (w & 1) * 8 + lane / 8;
    oa = (uint32_t)((lane / 8) * p.K + 8 * ((lane % 8) ^ swz<8>(r8))) * 2;
    if constexpr (AN) {
      const int r16 = (w & 3) * 4 + lane / 16;
      oa = (uint32_t)((lane / 16) * p.M + 8 * ((lane % 16) ^ swz<16>(r16))) * 2;
    }
    if constexpr (BN) {
      const int r16 = (w & 3) * 4 + lane / 16;
      ob = (uint32_t)((lane / 16) * p.N + 8 * ((lane % 16) ^ swz<16>(r16))) * 2;
    } else {
      ob = oa;
    }
  }
  auto issue = [&](int ks, int st) {
    const int k0 = kbeg + ks * TK;
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = 4 * j + w;
      if constexpr (AN)
        dma16(ra, uniform((int)(la + blk * 1024)), oa + (uint32_t)(((k0 + 4 * blk) * p.M + m0) * 2), 0u);
      else if (j < TM / 32)
        dma16(ra, uniform((int)(la + blk * 1024)), oa + (uint32_t)(((m0 + 8 * blk) * p.K + k0) * 2), 0u);
      if constexpr (BN)
        dma16(rb, uniform((int)(lb + blk * 1024)), ob + (uint32_t)(((k0 + 4 * blk) * p.N + n0) * 2), 0u);
      else if (j < TN / 32)
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

  f32x16 acc[NB][MB];  // [n block][m block]: register 4i + j of lane l = C[row l32][column 8i + 4half + j]
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < MB; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int nk = p.K / splits / TK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    if (ks + 1 < nk) issue(ks + 1, st ^ 1);  // the other stage was last read before the previous barrier
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
    bf16x8 bo[4][MB], ao[4][NB];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int y = 0; y < MB; ++y) {
        if constexpr (AN)
          bo[kk][y] = tr_op(la, MB * wm + y, kk);
        else
          bo[kk][y] = row_op(la, MB * wm + y, kk);
      }
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        if constexpr (BN)
          ao[kk][x] = tr_op(lb, NB * wn + x, kk);
        else
          ao[kk][x] = row_op(lb, NB * wn + x, kk);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int y = 0; y < MB; ++y) acc[x][y] = mfma32(ao[kk][x], bo[kk][y], acc[x][y]);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next stage have landed
    __syncthreads();
  }

  if (splits > 1) {  // fp32 partial tile, row-major 128 x 128
    float* dst = p.part + (((long)bz * splits + sp) * gemm_tiles(p.M, p.N, p.sym, TM, TN) + tile) * (TM * TN);
#pragma unroll
    for (int y = 0; y < MB; ++y)
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * (MB * wm + y) + l32, c = 32 * (NB * wn + x) + 8 * i + 4 * half;
          *(f32x4*)(dst + r * TN + c) = f32x4{acc[x][y][4 * i], acc[x][y][4 * i + 1], acc[x][y][4 * i + 2],
                                             acc[x][y][4 * i + 3]};
        }
    return;
  }

  // the diagonal of a symmetric product's diagonal tile (waves with wm == wn
  // hold its 32 x 32 diagonal blocks acc[y][y]): lane l has the element of
  // row l32 when its half matches, in register 4 (l32 >> 3) + (l32 & 3); the
  // wave adds them by a fixed butterfly
  if constexpr (TM == 128) {
    if (p.trace != nullptr && tm == tn && wm == wn) {
      const int rr = 4 * (l32 >> 3) + (l32 & 3);
      const bool on = half == ((l32 >> 2) & 1);
#pragma unroll
      for (int y = 0; y < MB; ++y) {
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) v = (on && r == rr) ? acc[y][y][r] : v;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
        if (lane == 0) p.trace[bz * gemm_trace_parts(p.M) + 4 * tm + MB * wm + y] = v;
      }
    }
  }

  // epilogue: C = alpha acc + beta C0 (bf16), mirrored for an off-diagonal tile of a symmetric product
  const long cbase = bz * p.M * p.N;
  float al, be;
  gemm_scales(p, bz, al, be);
#pragma unroll
  for (int y = 0; y < MB; ++y)
    gemm_store_rows(p, cbase, m0 + 32 * (MB * wm + y) + l32, n0 + 32 * NB * wn + 4 * half, acc, y, al, be,
                    p.sym && tm != tn);
}

// The 192 x 192 tile: four waves, each a 96 x 96 quarter (3 x 3 blocks of
// 32 x 32, nine accumulators), K in steps of 32 through three LDS stages
// (copies two steps ahead), two workgroups per compute unit. Per byte
// copied into LDS it does 1.5 times the MFMA work of the 128 x 128 tile,
// and at m = 768 its tile count matches the workgroup slots (512 per
// product of the trainer's groups: one full round).
// LDS: [x][k] operand tiles are 192 rows of 64 bytes (4 chunks), chunk j of
// row r at j ^ ((r >> 2) & 3), so that the 16 rows a read serves per pass
// at one logical chunk land on 16 distinct 16-byte bank groups. A [k][n]
// tile (B given as [K][N]) is three 64-column sub-tiles of 32 rows of 128
// bytes, swizzled as the 8-chunk rows above and read with transpose reads.
template <bool BN>
__global__ void __launch_bounds__(256, 2) gemm192_kernel(GemmParams p) {
  constexpr int T = 192, TK = 32, NST = 3;
  constexpr int SE = T * TK;  // elements per operand stage
  __shared__ __attribute__((aligned(1024))) bf16 As[NST][SE];
  __shared__ __attribute__((aligned(1024))) bf16 Bs[NST][SE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;  // row blocks 3 wm .., column blocks 3 wn ..
  const int tiles_n = p.N / T;
  const int per_mat = gemm_tiles(p.M, p.N, p.sym, T, T);
  const int w_item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  const int tile = w_item % per_mat;
  int tm, tn;
  tile_of(tile, tiles_n, p.sym, tm, tn);
  const int m0 = tm * T;
  const int n0 = tn * T;
  const long bz = w_item / per_mat;

  const bf16* A = (const bf16*)p.a + bz * p.M * p.K;
  const bf16* B = (const bf16*)p.b + bz * p.N * p.K;
  const u32x4 ra = rsrc_words(A, (uint32_t)(p.M * p.K * 2));
  const u32x4 rb = rsrc_words(B, (uint32_t)(p.N * p.K * 2));

  // Copies: instruction j (0..2) of wave w fills the 1 KB block blk = 4j + w
  // of each operand stage. [x][k]: rows 16 blk + lane/4, the lane's LDS chunk
  // lane % 4 holding global chunk (lane % 4) ^ ((lane >> 4) & 3) (the row's
  // swizzle: (row >> 2) & 3 = (lane >> 4) & 3). [k][n]: sub-tile j, k-rows
  // 8w + lane/8, LDS chunk lane % 8 holding column chunk (lane % 8) ^ swz<8>(row).
  const uint32_t ox = (uint32_t)((lane / 4) * p.K + 8 * ((lane & 3) ^ ((lane >> 4) & 3))) * 2;
  uint32_t obn = 0;
  if constexpr (BN) {
    const int kr = 8 * w + lane / 8;
    obn = (uint32_t)((lane / 8) * p.N + 8 * ((lane & 7) ^ swz<8>(kr))) * 2;
  }
  auto issue = [&](int ks, int st) {
    const int k0 = ks * TK;
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int blk = 4 * j + w;
      dma16(ra, uniform((int)(la + blk * 1024)), ox + (uint32_t)(((m0 + 16 * blk) * p.K + k0) * 2), 0u);
      if constexpr (BN)
        dma16(rb, uniform((int)(lb + blk * 1024)), obn + (uint32_t)(((k0 + 8 * w) * p.N + n0 + 64 * j) * 2), 0u);
      else
        dma16(rb, uniform((int)(lb + blk * 1024)), ox + (uint32_t)(((n0 + 16 * blk) * p.K + k0) * 2), 0u);
    }
  };

  // Row reads of [x][k] tiles: row 32 blk + l32, chunk 2 kk + half (k = 16 kk
  // + 8 half + e). Transpose reads of the [k][n] tile: column block cb (32
  // columns) is half cb % 2 of sub-tile cb / 2; rows 16 kk + 8 half + tq (+4),
  // columns 16 g1 + 4 qq of the block; lane l receives column l32 of the
  // block at k = 16 kk + 8 half + e, the same K order as the row reads.
  auto row_op = [&](uint32_t base, int blk, int kk) {
    const int r = 32 * blk + l32;
    return *(SA_LDS const bf16x8*)(uintptr_t)(base + (uint32_t)(r * 64 + (((2 * kk + half) ^ ((r >> 2) & 3)) << 4)));
  };
  uint32_t trb[2] = {0u, 0u};
  if constexpr (BN) {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) trb[hi] = (uint32_t)swz_off<8>(8 * half + tq + 4 * hi, 16 * g1 + 4 * qq) * 2;
  }
  auto tr_op = [&](uint32_t base, int cb, int kk) {
    const uint32_t rbase = base + (uint32_t)((cb >> 1) * 4096 + kk * 16 * 128);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (SA_LDS bf16x4*)(uintptr_t)(rbase + (trb[0] ^ (uint32_t)((cb & 1) << 6))));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (SA_LDS bf16x4*)(uintptr_t)(rbase + (trb[1] ^ (uint32_t)((cb & 1) << 6))));
    return cat(lo, hi);
  };

  f32x16 acc[3][3];  // [n block][m block]: register 4i + j of lane l = C[row l32][column 8i + 4half + j]
#pragma unroll
  for (int x = 0; x < 3; ++x)
#pragma unroll
    for (int y = 0; y < 3; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int nk = p.K / TK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  int st = 0;
#pragma clang loop unroll(disable)
  for (int ks = 0; ks < nk; ++ks) {
    // this wave's copies of step ks have landed (those of step ks + 1, six
    // instructions, may still be in flight); after the barrier every wave's
    // have, and every wave has finished step ks - 1, whose stage the copies
    // of step ks + 2 overwrite
    if (ks + 1 < nk)
      asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (ks + 2 < nk) issue(ks + 2, st == 0 ? 2 : st - 1);
    const uint32_t la = lds_addr(&As[st][0]);
    const uint32_t lb = lds_addr(&Bs[st][0]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 bo[3], ao[3];
#pragma unroll
      for (int y = 0; y < 3; ++y) bo[y] = row_op(la, 3 * wm + y, kk);
#pragma unroll
      for (int x = 0; x < 3; ++x) {
        if constexpr (BN)
          ao[x] = tr_op(lb, 3 * wn + x, kk);
        else
          ao[x] = row_op(lb, 3 * wn + x, kk);
      }
#pragma unroll
      for (int x = 0; x < 3; ++x)
#pragma unroll
        for (int y = 0; y < 3; ++y) acc[x][y] = mfma32(ao[x], bo[y], acc[x][y]);
    }
    st = st == 2 ? 0 : st + 1;
  }

  // epilogue: C = alpha acc + beta C0 (bf16), mirrored for an off-diagonal tile of a symmetric product
  const long cbase = bz * p.M * p.N;
  float al, be;
  gemm_scales(p, bz, al, be);
#pragma unroll
  for (int y = 0; y < 3; ++y)
    gemm_store_rows(p, cbase, m0 + 32 * (3 * wm + y) + l32, n0 + 32 * 3 * wn + 4 * half, acc, y, al, be,
                    p.sym && tm != tn);
}

// Split-K reduction: the 32 x 32 block blockIdx.x % 16 of computed tile
// blockIdx.x / 16 of matrix blockIdx.y. Thread (r, q) adds the partials of
// row r, columns 4q .. 4q + 3 in split order, applies alpha and beta and
// stores 8 bytes; the mirror goes through an LDS transpose.
__global__ void __launch_bounds__(256) gemm_reduce_kernel(GemmParams p) {
  __shared__ unsigned short t[32][34];
  __shared__ float dg[32];
  const int tile = blockIdx.x / 16, br = (blockIdx.x / 4) & 3, bc = blockIdx.x & 3;
  int tm, tn;
  tile_of(tile, p.N / 128, p.sym, tm, tn);
  const long bz = blockIdx.y;
  const int ntile = gemm_tiles(p.M, p.N, p.sym);
  const int r = threadIdx.x >> 3, q = threadIdx.x & 7;
  const int lr = 32 * br + r, lc = 32 * bc + 4 * q;  // within the 128 x 128 tile
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.splits; ++s) {
    const f32x4 x = *(const f32x4*)(p.part + (((long)bz * p.splits + s) * ntile + tile) * (128 * 128) + lr * 128 + lc);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += x[e];
  }
  // a diagonal block's diagonal (element (r, 4q + e) with 4q + e = r), added in row order
  if (p.trace != nullptr && tm == tn && br == bc) {
    const int e = r - 4 * q;
    if (e >= 0 && e < 4) dg[r] = e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : v[3];
    __syncthreads();
    if (threadIdx.x == 0) {
      float s = 0.f;
      for (int i = 0; i < 32; ++i) s += dg[i];
      p.trace[bz * gemm_trace_parts(p.M) + 4 * tm + br] = s;
    }
  }
  const long row = tm * 128 + lr, col = tn * 128 + lc;
  const long off = bz * p.M * p.N + row * p.N + col;
  float al, be;
  gemm_scales(p, bz, al, be);
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = al * v[e];
  if (p.c0 != nullptr) {
    const u32x2 c0 = *(const u32x2*)((const bf16*)p.c0 + off);
    o[0] += be * __uint_as_float(c0[0] << 16);
    o[1] += be * __uint_as_float(c0[0] & 0xffff0000u);
    o[2] += be * __uint_as_float(c0[1] << 16);
    o[3] += be * __uint_as_float(c0[1] & 0xffff0000u);
  }
  u32x2 w;
  w[0] = pack2(o[0], o[1]);
  w[1] = pack2(o[2], o[3]);
  *(u32x2*)((bf16*)p.c + off) = w;
  if (!(p.sym && tm != tn)) return;
  t[r][4 * q] = (unsigned short)(w[0] & 0xffffu);
  t[r][4 * q + 1] = (unsigned short)(w[0] >> 16);
  t[r][4 * q + 2] = (unsigned short)(w[1] & 0xffffu);
  t[r][4 * q + 3] = (unsigned short)(w[1] >> 16);
  __syncthreads();
  // mirror: row (block column r) of the transposed block, its columns 4q .. 4q + 3 = block rows
  u32x2 m;
  m[0] = (uint32_t)t[4 * q][r] | ((uint32_t)t[4 * q + 1][r] << 16);
  m[1] = (uint32_t)t[4 * q + 2][r] | ((uint32_t)t[4 * q + 3][r] << 16);
  const long moff = bz * p.M * p.N + (long)(tn * 128 + 32 * bc + r) * p.M + tm * 128 + 32 * br + 4 * q;
  *(u32x2*)((bf16*)p.c + moff) = m;
}

hipError_t launch_gemm(const GemmParams& p, bool b_kn, int batch, hipStream_t stream, int tile, bool a_kn) {
  const int splits = p.splits > 1 ? p.splits : 1;
  if (a_kn) {
    if (!b_kn || tile != 128) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(gemm_tiles(p.M, p.N, p.sym) * splits * batch));
    hipLaunchKernelGGL((gemm_kernel<true, 128, true>), grid, dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)(gemm_tiles(p.M, p.N, p.sym) * 16), (unsigned)batch),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (p.trace != nullptr && (tile != 128 || b_kn || !p.sym)) return hipErrorInvalidValue;
  if (tile == 192) {
    if (splits > 1 || p.M % 192 != 0 || p.N % 192 != 0 || p.K % 32 != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(gemm_tiles(p.M, p.N, p.sym, 192, 192) * batch));
    if (b_kn)
      hipLaunchKernelGGL((gemm192_kernel<true>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm192_kernel<false>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (tile == 64) {
    if (b_kn || splits > 1 || p.M % 64 != 0 || p.N % 64 != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(gemm_tiles(p.M, p.N, p.sym, 64, 64) * batch));
    hipLaunchKernelGGL((gemm_kernel<false, 64>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (tile != 128 && (tile != 96 || !b_kn || splits > 1 || p.sym || p.M % 96 != 0)) return hipErrorInvalidValue;
  const int ntile = gemm_tiles(p.M, p.N, p.sym, tile);
  const dim3 grid((unsigned)(ntile * splits * batch));
  if (tile == 96)
    hipLaunchKernelGGL((gemm_kernel<true, 96>), grid, dim3(256), 0, stream, p);
  else if (b_kn)
    hipLaunchKernelGGL((gemm_kernel<true, 128>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<false, 128>), grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)(ntile * 16), (unsigned)batch), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
