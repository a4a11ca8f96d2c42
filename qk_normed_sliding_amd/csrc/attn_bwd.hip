// Backward of QK-normed, grouped-query, sliding-window causal attention (gfx950).
//
// Gradients of the layer in attn_fwd.hip with respect to the raw q, k, v:
//   P_ij    = exp(S_ij - LSE_i)            (row statistics from the forward)
//   Delta_i = <dO_i, O_i>
//   dV_j   += sum_i P_ij dO_i              (summed over the query heads of a group)
//   dS_ij   = P_ij (<dO_i, v_j> - Delta_i)
//   dq_hat  = scale dS K_hat,  dk_hat = scale dS^T Q_hat (summed over the group)
//   dx      = r (dx_hat - x_hat <dx_hat, x_hat> / D)   (RMS-norm backward)
// Sources: [post] QK-norm and SSSL passages; [guide] 8.2.1 (RMSNorm, GQA,
// sliding window). The backward is the derivative of that forward.
//
// Three kernels:
//   1. pre-pass, one pass over the rows: Delta = rowsum(dO * O), the normed
//      rows q_hat (bf16, so the main loop stages Q tiles without arithmetic)
//      and zeroing of the fp32 dQ accumulator;
//   2. main: one workgroup per (batch, KV head, 128-key block); 4 waves own
//      32 keys each and keep K_hat, V and the dK/dV accumulators in registers
//      while streaming every (query head of the group, 64-row query block) of
//      the band through LDS. Q_hat/dO tiles are prefetched into registers one
//      block ahead and double-buffered in LDS (XOR-swizzled rows: both the
//      16-byte operand reads and the transpose reads are bank-conflict free).
//      S and dP come out with one key per lane; P and dS then feed
//      dV^T += dO^T P and dK^T += Q_hat^T dS directly (operands dO^T and
//      Q_hat^T via the LDS transpose read). dS goes to LDS once and the
//      workgroup adds its dQ_hat contribution for all 128 keys to the fp32
//      accumulator with buffer float atomics;
//   3. finalize: dq = norm-backward(scale * dQ_hat) -> bf16.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

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

// ---------------------------------------------------------------- pre-pass
template <int D, bool NORM>
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(BwdParams p) {
  constexpr int CPR = D / 8;           // 16-byte bf16 chunks per row
  constexpr int RPB = 256 / CPR;       // rows per block iteration
  const long rows = (long)p.B * p.T * p.Hq;
  const int sub = threadIdx.x % CPR;
  for (long row = (long)blockIdx.x * RPB + threadIdx.x / CPR; row < rows; row += (long)gridDim.x * RPB) {
    float a[8], c[8];
    unpack8(ld16((const bf16*)p.dout + row * D + 8 * sub), a);
    unpack8(ld16((const bf16*)p.o + row * D + 8 * sub), c);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += a[e] * c[e];
    s = group_sum<CPR>(s);
    if constexpr (NORM) {
      float x[8];
      unpack8(ld16((const bf16*)p.q + row * D + 8 * sub), x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= r;
      st16((bf16*)p.qhat + row * D + 8 * sub, pack8(x));
    }
    float* acc = p.dq_acc + row * D + 8 * sub;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)acc = z;
    *(f32x4*)(acc + 4) = z;
    if (sub == 0) {
      const int h = (int)(row % p.Hq);
      const long bt = row / p.Hq;
      const int t = (int)(bt % p.T);
      const int b = (int)(bt / p.T);
      p.delta[((long)b * p.Hq + h) * p.T + t] = s;
    }
  }
}

// ---------------------------------------------------------------- main
template <int D, int BQ, bool NORM>
__global__ void __launch_bounds__(256, 1) attn_bwd_kernel(BwdParams p) {
  constexpr int NW = 4;
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;        // keys per workgroup
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per head row
  constexpr int KSP = D + 32;        // K_hat row pitch (bf16): transpose reads of 4 rows hit disjoint banks
  constexpr int NQC = BQ / 32;       // 32-row query chunks per block
  constexpr int DCH = BQ / 8;        // 16-byte chunks per dS row (one row per key)
  constexpr int NBLK = NQC * NDB;    // 32x32 blocks of the dQ tile
  constexpr int BPW = NBLK / NW;     // dQ blocks per wave
  constexpr int QCPT = BQ * CPR / NT;  // Q_hat (and dO) chunks per thread per block
  static_assert(NBLK % NW == 0, "dQ tile must split evenly over the waves");
  static_assert((BK * CPR) % NT == 0 && (BQ * CPR) % NT == 0, "tiles must split evenly");
  static_assert(CPR == 16 || CPR == 8, "head_dim 64 or 128");
  static_assert(DCH == 8, "dS rows of 64 queries");

  __shared__ __attribute__((aligned(16))) bf16 Ks[BK * KSP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 dSs[BK * BQ];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dls[2][BQ];
  __shared__ float rks[BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;

  // key blocks in ascending order: the first blocks see the most queries
  const int bid = blockIdx.x;
  const int kb = bid / (p.B * p.Hkv);
  const int g = (bid / p.B) % p.Hkv;
  const int b = bid % p.B;
  const int kb0 = kb * BK;
  const int kw0 = kb0 + 32 * wave;  // first key of this wave
  const int key = kw0 + l32;

  // ---- K_hat block into LDS (RMS-normed), rstd per key; V fragment from global
  {
    const bf16* kb_ptr = (const bf16*)p.k + ((long)b * T * p.Hkv + g) * D + (long)kb0 * kvstride;
    const auto rk = make_rsrc(kb_ptr, (uint32_t)max(0, T - kb0) * kvstride * 2);
#pragma unroll
    for (int i = 0; i < BK * CPR / NT; ++i) {
      const int c = tid + NT * i;
      const int kt = c / CPR;
      const int col = 8 * (c % CPR);
      u32x4 w = bload16(rk, (uint32_t)(kt * kvstride + col) * 2);
      if constexpr (NORM) {
        float x[8];
        unpack8(w, x);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= r;
        w = pack8(x);
        if (c % CPR == 0) rks[kt] = r;
      }
      *(u32x4*)&Ks[kt * KSP + col] = w;
    }
  }
  bf16x8 vf[KST];
  {
    const bf16* vb_ptr = (const bf16*)p.v + ((long)b * T * p.Hkv + g) * D + (long)kb0 * kvstride;
    const auto rv = make_rsrc(vb_ptr, (uint32_t)max(0, T - kb0) * kvstride * 2);
    const uint32_t off = (uint32_t)((32 * wave + l32) * kvstride + 8 * half) * 2;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) vf[kk] = __builtin_bit_cast(bf16x8, bload16(rv, off + 32 * kk));
  }
  __syncthreads();
  bf16x8 kf[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) kf[kk] = *(const bf16x8*)&Ks[(32 * wave + l32) * KSP + 16 * kk + 8 * half];

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv_acc[db][r] = 0.f;
      dk_acc[db][r] = 0.f;
    }

  // query blocks whose rows can see at least one key of this block
  const int q_hi = (W < 0) ? T - 1 : min(T - 1, kb0 + BK - 1 + W);
  const int qb_lo = kb0 / BQ;
  const int nqb = q_hi / BQ - qb_lo + 1;
  const int nit = p.G * nqb;

  // ---- lane parts of the LDS addresses (element offsets)
  const int tq = (lane >> 2) & 3;              // transpose read: row within a group of 4
  const int g1 = (lane >> 4) & 1;              // transpose read: 16-column half
  const int qq = lane & 3;                     // transpose read: 4-column quad
  // 16-byte A-operand reads of Q_hat / dO rows 32qc + swap23(l32), chunk 2kk + half
  int a_off[KST];
  {
    const int r = swap23(l32);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) a_off[kk] = swz_off<CPR>(r, 16 * kk + 8 * half);
  }
  // transpose reads of Q_hat / dO rows 32qc + 16ks + 8half + tq (+4), columns 32db + 16g1 + 4qq
  int t_off[2][NDB];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < NDB; ++db) t_off[hi][db] = swz_off<CPR>(8 * half + tq + 4 * hi, 32 * db + 16 * g1 + 4 * qq);
  // dS rows (keys) written by this lane: row 32w + l32, chunk 4qc + 2ks + half
  const int ds_row = 32 * wave + l32;
  // transpose reads of dS rows 16ks + 8half + tq (+4), columns 32qc + 16g1 + 4qq
  int dt_off[2][NQC];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int qc = 0; qc < NQC; ++qc) dt_off[hi][qc] = swz_off<DCH>(8 * half + tq + 4 * hi, 32 * qc + 16 * g1 + 4 * qq);
  const int k_tr = (8 * half + tq) * KSP + 16 * g1 + 4 * qq;

  // ---- prefetch of one (head, query block) step into registers
  u32x4 qreg[QCPT], oreg[QCPT];
  float lreg = 0.f;
  auto prefetch = [&](int it) {
    const int hh = it / nqb;
    const int qb = qb_lo + it % nqb;
    const int head = g * p.G + hh;
    const int row0 = qb * BQ;
    const long first = ((long)b * T + row0) * qstride + (long)head * D;
    const uint32_t bytes = (uint32_t)max(0, T - row0) * qstride * 2;
    const auto rq = make_rsrc((const bf16*)p.qhat + first, bytes);
    const auto rd = make_rsrc((const bf16*)p.dout + first, bytes);
#pragma unroll
    for (int i = 0; i < QCPT; ++i) {
      const int c = tid + NT * i;
      const uint32_t off = (uint32_t)((c / CPR) * qstride + 8 * (c % CPR)) * 2;
      qreg[i] = bload16(rq, off);
      oreg[i] = bload16(rd, off);
    }
    if (tid < 2 * BQ) {
      const int rr = row0 + (tid % BQ);
      const float* src = (tid < BQ ? p.lse : p.delta) + ((long)b * p.Hq + head) * T;
      lreg = rr < T ? src[rr] : (tid < BQ ? INFINITY : 0.f);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QCPT; ++i) {
      const int c = tid + NT * i;
      const int o = swz_off<CPR>(c / CPR, 8 * (c % CPR));
      *(u32x4*)&Qs[buf][o] = qreg[i];
      *(u32x4*)&dOs[buf][o] = oreg[i];
    }
    if (tid < BQ) lse2s[buf][tid] = lreg * kLog2e;
    else if (tid < 2 * BQ) dls[buf][tid - BQ] = lreg;
  };

  // ---- one step: S, dP, P, dS, dV, dK for this wave's 32 keys; dS to LDS
  auto compute = [&](int buf, int row0) {
    const bf16* Qb = Qs[buf];
    const bf16* Ob = dOs[buf];
#pragma unroll
    for (int qc = 0; qc < NQC; ++qc) {
      const int q0 = row0 + 32 * qc;
      const bool act = !(q0 + 31 < kw0 || (W >= 0 && q0 > kw0 + 31 + W));
      if (!act) continue;
      const bool edge = !(q0 >= kw0 + 31 && (W < 0 || q0 + 31 - kw0 <= W)) || q0 + 31 >= T;
      const bf16* qa = Qb + 32 * qc * D;
      const bf16* oa = Ob + 32 * qc * D;
      bf16x8 qv[KST], ov[KST];
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) {
        qv[kk] = *(const bf16x8*)(qa + a_off[kk]);
        ov[kk] = *(const bf16x8*)(oa + a_off[kk]);
      }
      f32x16 s = mfma32(qv[0], kf[0], f32x16{});
      f32x16 dp = mfma32(ov[0], vf[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < KST; ++kk) {
        s = mfma32(qv[kk], kf[kk], s);
        dp = mfma32(ov[kk], vf[kk], dp);
      }
      // register r of this lane: query q0 + 16(r>>3) + 8half + (r&7), key `key`
      float pr[16], ds[16];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int qo = 32 * qc + 16 * ks + 8 * half;
        const f32x4 l0 = *(const f32x4*)&lse2s[buf][qo];
        const f32x4 l1 = *(const f32x4*)&lse2s[buf][qo + 4];
        const f32x4 d0 = *(const f32x4*)&dls[buf][qo];
        const f32x4 d1 = *(const f32x4*)&dls[buf][qo + 4];
        const uint32_t rk = (uint32_t)(q0 + 16 * ks + 8 * half - key);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * ks + e;
          const float lv = e < 4 ? l0[e] : l1[e - 4];
          const float dv = e < 4 ? d0[e] : d1[e - 4];
          float pe = fast_exp2(__builtin_fmaf(s[r], p.c1, -lv));
          if (edge) pe = (rk + (uint32_t)e <= Wm) ? pe : 0.f;
          pr[r] = pe;
          ds[r] = pe * (dp[r] - dv);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pack8(pr + 8 * ks));
        const u32x4 dsw = pack8(ds + 8 * ks);
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, dsw);
        const int rbase = (32 * qc + 16 * ks) * D;
        bf16x4 a_lo[NDB], a_hi[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          a_lo[db] = lds_read_tr(Ob + rbase + t_off[0][db]);
          a_hi[db] = lds_read_tr(Ob + rbase + t_off[1][db]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) dv_acc[db] = mfma32(cat(a_lo[db], a_hi[db]), pb, dv_acc[db]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          a_lo[db] = lds_read_tr(Qb + rbase + t_off[0][db]);
          a_hi[db] = lds_read_tr(Qb + rbase + t_off[1][db]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) dk_acc[db] = mfma32(cat(a_lo[db], a_hi[db]), dsb, dk_acc[db]);
        // dS of this lane's key: 8 consecutive queries 32qc + 16ks + 8half + 0..7
        *(u32x4*)&dSs[swz_off<DCH>(ds_row, 32 * qc + 16 * ks + 8 * half)] = dsw;
      }
    }
  };

  // ---- dQ_hat[q][d] += sum_key dS[q][key] K_hat[key][d] over the 128 keys (unscaled)
  auto dq_gemm = [&](int it) {
    const int hh = it / nqb;
    const int qb = qb_lo + it % nqb;
    const int head = g * p.G + hh;
    const int row0 = qb * BQ;
    float* base = p.dq_acc + ((long)b * T * p.Hq + head) * D;
    const auto racc = make_rsrc(base, (uint32_t)T * qstride * 4);
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = wave * BPW + bi;
      const int qc = blk / NDB;
      const int db = blk % NDB;
      const int q0 = row0 + 32 * qc;
      f32x16 acc = {};
      bool any = false;
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int kw = kb0 + 32 * (ks / 2);  // first key of the wave that wrote these dS rows
        const bool act = !(q0 + 31 < kw || (W >= 0 && q0 > kw + 31 + W));
        if (!act) continue;
        any = true;
        const bf16* ap = dSs + 16 * ks * BQ;
        const bf16* bp = Ks + 16 * ks * KSP + 32 * db + k_tr;
        const bf16x8 a = cat(lds_read_tr(ap + dt_off[0][qc]), lds_read_tr(ap + dt_off[1][qc]));
        const bf16x8 bb = cat(lds_read_tr(bp), lds_read_tr(bp + 4 * KSP));
        acc = mfma32(a, bb, acc);
      }
      if (!any) continue;
      // accumulator: column = head_dim 32db + l32, row = query q0 + 8i + 4half + j.
      // The scalar offset is outside the descriptor's range check, so rows are
      // only put there when the whole chunk lies before T.
      const uint32_t voff = (uint32_t)((q0 + 4 * half) * qstride + 32 * db + l32) * 4;
      if (q0 + 31 < T) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], racc, voff,
                                                          (8 * (r >> 2) + (r & 3)) * qstride * 4, 0);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qo = 8 * (r >> 2) + (r & 3);
          if (q0 + 4 * half + qo < T)
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], racc, voff + qo * qstride * 4, 0, 0);
        }
      }
    }
  };

  prefetch(0);
  stage(0);
  __syncthreads();
  auto step = [&](int buf, int it) {
    const bool more = it + 1 < nit;
    if (more) prefetch(it + 1);
    compute(buf, (qb_lo + it % nqb) * BQ);
    __syncthreads();  // dS complete
    dq_gemm(it);
    if (more) stage(buf ^ 1);
    __syncthreads();  // next block staged; dS reads done
  };
  for (int it = 0; it < nit; it += 2) {
    step(0, it);
    if (it + 1 >= nit) break;
    step(1, it + 1);
  }

  // ---- epilogue: dv, and dk through the norm backward
  if (key >= T) return;
  bf16* dvp = (bf16*)p.dv + ((long)b * T + key) * kvstride + (long)g * D + 4 * half;
  bf16* dkp = (bf16*)p.dk + ((long)b * T + key) * kvstride + (long)g * D + 4 * half;
  float rk = 1.f, dot = 0.f;
  float kx[NDB][16];
  if constexpr (NORM) {
    rk = rks[32 * wave + l32];
    const bf16* kp = (const bf16*)p.k + ((long)b * T + key) * kvstride + (long)g * D + 4 * half;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 w = *(const u32x2*)(kp + 32 * db + 8 * i);
        kx[db][4 * i + 0] = __uint_as_float(w[0] << 16) * rk;
        kx[db][4 * i + 1] = __uint_as_float(w[0] & 0xffff0000u) * rk;
        kx[db][4 * i + 2] = __uint_as_float(w[1] << 16) * rk;
        kx[db][4 * i + 3] = __uint_as_float(w[1] & 0xffff0000u) * rk;
#pragma unroll
        for (int j = 0; j < 4; ++j) dot += p.scale * dk_acc[db][4 * i + j] * kx[db][4 * i + j];
      }
    dot = pair_sum(dot) * (1.f / D);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float dkv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g_hat = p.scale * dk_acc[db][4 * i + j];
        dkv[j] = NORM ? rk * (g_hat - kx[db][4 * i + j] * dot) : g_hat;
      }
      u32x2 wv, wk;
      wv[0] = pack2(dv_acc[db][4 * i], dv_acc[db][4 * i + 1]);
      wv[1] = pack2(dv_acc[db][4 * i + 2], dv_acc[db][4 * i + 3]);
      wk[0] = pack2(dkv[0], dkv[1]);
      wk[1] = pack2(dkv[2], dkv[3]);
      *(u32x2*)(dvp + 32 * db + 8 * i) = wv;
      *(u32x2*)(dkp + 32 * db + 8 * i) = wk;
    }
}

// ---------------------------------------------------------------- dq finalize
template <int D, bool NORM>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(BwdParams p) {
  constexpr int CPR = D / 8;
  constexpr int RPB = 256 / CPR;
  const long rows = (long)p.B * p.T * p.Hq;
  const int sub = threadIdx.x % CPR;
  for (long row = (long)blockIdx.x * RPB + threadIdx.x / CPR; row < rows; row += (long)gridDim.x * RPB) {
    const float* acc = p.dq_acc + row * D + 8 * sub;
    const f32x4 a0 = *(const f32x4*)acc;
    const f32x4 a1 = *(const f32x4*)(acc + 4);
    float g[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] *= p.scale;
    if constexpr (NORM) {
      float x[8];
      unpack8(ld16((const bf16*)p.q + row * D + 8 * sub), x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
      const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] *= r;
        dot += g[e] * x[e];
      }
      dot = group_sum<CPR>(dot) * (1.f / D);
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = r * (g[e] - x[e] * dot);
    }
    st16((bf16*)p.dq + row * D + 8 * sub, pack8(g));
  }
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, bool qk_norm, hipStream_t stream, const TimingEvents& ev) {
  constexpr int BQ = 64;
  const long rows = (long)p.B * p.T * p.Hq;
  const int rpb = 256 / (D / 8);
  const long nblk = (rows + rpb - 1) / rpb;
  const unsigned row_blocks = (unsigned)(nblk < 65536L ? nblk : 65536L);
  if (qk_norm)
    hipLaunchKernelGGL((attn_bwd_pre_kernel<D, true>), dim3(row_blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_pre_kernel<D, false>), dim3(row_blocks), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(p.nkb * p.B * p.Hkv));
  if (ev.start != nullptr && (e = hipEventRecord(ev.start, stream)) != hipSuccess) return e;
  if (qk_norm)
    hipLaunchKernelGGL((attn_bwd_kernel<D, BQ, true>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_kernel<D, BQ, false>), grid, dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev.stop != nullptr && (e = hipEventRecord(ev.stop, stream)) != hipSuccess) return e;
  if (qk_norm)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, true>), dim3(row_blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, false>), dim3(row_blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool qk_norm, hipStream_t stream, const TimingEvents& ev) {
  return head_dim == 128 ? launch_bwd_d<128>(p, qk_norm, stream, ev) : launch_bwd_d<64>(p, qk_norm, stream, ev);
}

}  // namespace sa
