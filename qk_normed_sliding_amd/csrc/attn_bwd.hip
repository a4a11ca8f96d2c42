// Backward of QK-normed, grouped-query, sliding-window causal attention (gfx950).
//
// Gradients of the layer in attn_fwd.hip with respect to the raw q, k, v:
//   P_ij    = exp(S_ij - LSE_i)            (row statistics from the forward)
//   Delta_i = <dO_i, O_i>
//   dV_j    = sum_{h in group} sum_i P_ij dO_i
//   dS_ij   = P_ij (<dO_i, v_j> - Delta_i)
//   dq_hat  = scale dS K_hat,  dk_hat = scale sum_{h in group} dS^T Q_hat
//   dx      = r (dx_hat - x_hat <dx_hat, x_hat> / D)   (RMS-norm backward)
// Sources: [post] QK-norm and SSSL passages; [guide] 8.2.1 (RMSNorm, GQA,
// sliding window). The backward is the derivative of that forward.
//
// Two kernels, no atomics:
//   1. dQ kernel, shaped like the forward (one workgroup per 128-row query
//      block of the query heads sharing a KV head, 32 rows per wave, Q_hat and
//      dO in registers, K_hat/V tiles of the band streamed through LDS):
//      recomputes S and dP, forms dS and accumulates dQ_hat^T = K_hat^T dS^T
//      with K_hat read K-major by the LDS transpose read. Its prologue
//      normalises the q rows (and writes q_hat for the second kernel) and
//      computes Delta from the dO and O rows; its epilogue applies the
//      RMS-norm backward and writes dq.
//   2. dK/dV kernel (one workgroup per 128-key block of a KV head; 4 waves
//      own 32 keys each and keep K_hat, V and the dK/dV accumulators in
//      registers): streams every (query head of the group, 64-row query
//      block) of the band through double-buffered, XOR-swizzled LDS, one
//      block ahead. S and dP come out with one key per lane; P and dS feed
//      dV^T += dO^T P and dK^T += Q_hat^T dS directly, with dO^T and Q_hat^T
//      read by the LDS transpose read. The GQA sum over the group's query
//      heads happens in the accumulators.
// Recomputing S and dP in both kernels costs 4 D MFMA FLOP per visible pair
// more than a single kernel with dQ atomics, but removes the fp32 atomic
// traffic, the dQ accumulator and its zeroing and finalize passes.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

// ---------------------------------------------------------------- dQ kernel
template <int D, int HPW, int BN, bool NORM>
__global__ void __launch_bounds__(HPW * 4 * 64) attn_bwd_dq_kernel(BwdParams p) {
  constexpr int WPH = 4;             // waves per head
  constexpr int BM = WPH * 32;       // query rows per block
  constexpr int NT = HPW * WPH * 64;
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int VP = D + 8;          // V row pitch (bf16): 16-byte reads of 16 rows hit 16 bank groups
  constexpr int CPT = BN * CPR / NT;
  constexpr int NCH = BN / 32;
  static_assert(CPT >= 1 && (BN * CPR) % NT == 0, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * D];   // K_hat, XOR-swizzled rows
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int per_qb = p.B * p.Hkv * p.nsub;
  const int bid = blockIdx.x;
  const int qb = p.nqb - 1 - bid / per_qb;  // heavy query blocks first
  int rem = bid % per_qb;
  const int sub = rem % p.nsub;
  rem /= p.nsub;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const int head = g * p.G + sub * HPW + wave / WPH;
  const int r0 = qb * BM + (wave % WPH) * 32;
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;
  const bool wave_active = r0 < T;
  const int row = r0 + l32;

  // ---- prologue: q_hat and dO fragments (B operands), Delta, LSE of this lane's row
  bf16x8 qf[KST], df[KST];
  float r_q = 1.f, delta, lse2;
  {
    const long first = ((long)b * T * p.Hq + head) * D;
    const uint32_t bytes = (uint32_t)T * qstride * 2;
    const auto rq = make_rsrc((const bf16*)p.q + first, bytes);
    const auto rd = make_rsrc((const bf16*)p.dout + first, bytes);
    const auto ro = make_rsrc((const bf16*)p.o + first, bytes);
    const uint32_t off = (uint32_t)(row * qstride + 8 * half) * 2;
    float x[KST][8];
    float ss = 0.f, dd = 0.f;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      unpack8(bload16(rq, off + 32 * kk), x[kk]);
      const u32x4 dw = bload16(rd, off + 32 * kk);
      df[kk] = __builtin_bit_cast(bf16x8, dw);
      float dv[8], ov[8];
      unpack8(dw, dv);
      unpack8(bload16(ro, off + 32 * kk), ov);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += x[kk][e] * x[kk][e];
        dd += dv[e] * ov[e];
      }
    }
    delta = pair_sum(dd);
    if constexpr (NORM) r_q = fast_rsqrt(pair_sum(ss) * (1.f / D) + p.eps);
    bf16* qh = (bf16*)p.qhat + first + (long)row * qstride + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kk][e] *= r_q;
      const u32x4 w = pack8(x[kk]);
      qf[kk] = __builtin_bit_cast(bf16x8, w);
      if (NORM && row < T) st16(qh + 16 * kk, w);
    }
    const long lrow = ((long)b * p.Hq + head) * T + row;
    lse2 = row < T ? p.lse[lrow] * kLog2e : INFINITY;
    if (half == 0 && row < T) p.delta[lrow] = delta;
  }

  // ---- key tiles that intersect the band of this block's rows
  const int row_lo = qb * BM;
  const int row_hi = min(T, row_lo + BM) - 1;
  const int key_lo = (W < 0) ? 0 : max(0, row_lo - W);
  const int n_lo = key_lo / BN;
  const int n_hi = row_hi / BN;

  const bf16* kbase = (const bf16*)p.k + ((long)b * T * p.Hkv + g) * D;
  const bf16* vbase = (const bf16*)p.v + ((long)b * T * p.Hkv + g) * D;
  uint32_t ld_off[CPT];
  int st_k[CPT], st_v[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    ld_off[i] = (uint32_t)((c / CPR) * kvstride + 8 * (c % CPR)) * 2;
    st_k[i] = swz_off<CPR>(c / CPR, 8 * (c % CPR));
    st_v[i] = (c / CPR) * VP + 8 * (c % CPR);
  }
  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int n) {
    const long first = (long)n * BN * kvstride;
    const uint32_t bytes = (uint32_t)max(0, T - n * BN) * kvstride * 2;
    const auto rk = make_rsrc(kbase + first, bytes);
    const auto rv = make_rsrc(vbase + first, bytes);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      kreg[i] = bload16(rk, ld_off[i]);
      vreg[i] = bload16(rv, ld_off[i]);
    }
  };
  auto store_tile = [&](bf16* Kd, bf16* Vd) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      u32x4 kw = kreg[i];
      if constexpr (NORM) {
        float x[8];
        unpack8(kw, x);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= r;
        kw = pack8(x);
      }
      *(u32x4*)(Kd + st_k[i]) = kw;
      *(u32x4*)(Vd + st_v[i]) = vreg[i];
    }
  };

  // lane parts of the LDS addresses
  int ka_off[KST];  // 16-byte reads of K_hat rows 32c + swap23(l32), chunk 2kk + half
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) ka_off[kk] = swz_off<CPR>(swap23(l32), 16 * kk + 8 * half);
  const int v_lane = swap23(l32) * VP + 8 * half;
  int kt_off[2][NDB];  // transpose reads of K_hat rows 32c + 16ks + 8half + tq (+4), cols 32db + 16g1 + 4qq
  {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < NDB; ++db) kt_off[hi][db] = swz_off<CPR>(8 * half + tq + 4 * hi, 32 * db + 16 * g1 + 4 * qq);
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  auto chunk = [&](const bf16* Kb, const bf16* Vb, int n, int c, bool edge) {
    bf16x8 ka[KST], va[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      ka[kk] = *(const bf16x8*)(Kb + 32 * c * D + ka_off[kk]);
      va[kk] = *(const bf16x8*)(Vb + 32 * c * VP + v_lane + 16 * kk);
    }
    f32x16 s = mfma32(ka[0], qf[0], f32x16{});
    f32x16 dp = mfma32(va[0], df[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < KST; ++kk) {
      s = mfma32(ka[kk], qf[kk], s);
      dp = mfma32(va[kk], df[kk], dp);
    }
    // register r: key n*BN + 32c + 16(r>>3) + 8half + (r&7), query `row`
    float ds[16];
    const uint32_t rk = (uint32_t)(row - (n * BN + 32 * c + 8 * half));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pe = fast_exp2(__builtin_fmaf(s[r], p.c1, -lse2));
      if (edge) pe = (rk - (uint32_t)(16 * (r >> 3) + (r & 7)) <= Wm) ? pe : 0.f;
      ds[r] = pe * (dp[r] - delta);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, pack8(ds + 8 * ks));
      const bf16* kp = Kb + (32 * c + 16 * ks) * D;
      bf16x4 lo[NDB], hi[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        lo[db] = lds_read_tr(kp + kt_off[0][db]);
        hi[db] = lds_read_tr(kp + kt_off[1][db]);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = mfma32(cat(lo[db], hi[db]), dsb, dq[db]);
    }
  };
  auto tile = [&](const bf16* Kb, const bf16* Vb, int n) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int kc = n * BN + 32 * c;
      const bool act = !(kc > r0 + 31 || (W >= 0 && kc + 31 < r0 - W));
      const bool edge = !(kc + 31 <= r0 && (W < 0 || r0 + 31 - kc <= W));
      if (act) chunk(Kb, Vb, n, c, edge);
    }
  };
  auto step = [&](const bf16* Kb, const bf16* Vb, bf16* Kn, bf16* Vn, int n) {
    const bool more = n < n_hi;
    if (more) load_tile(n + 1);
    if (wave_active) tile(Kb, Vb, n);
    if (more) store_tile(Kn, Vn);
    __syncthreads();
  };
  load_tile(n_lo);
  store_tile(Ks[0], Vs[0]);
  __syncthreads();
  for (int n = n_lo; n <= n_hi; n += 2) {
    step(Ks[0], Vs[0], Ks[1], Vs[1], n);
    if (n + 1 > n_hi) break;
    step(Ks[1], Vs[1], Ks[0], Vs[0], n + 1);
  }

  // ---- epilogue: dq = r (dq_hat - q_hat <dq_hat, q_hat> / D), dq_hat = scale * acc.
  // The accumulator holds head_dim 32db + 8i + 4half + j of this lane's row.
  if (!wave_active || row >= T) return;
  const long rowoff = ((long)b * T + row) * qstride + (long)head * D + 4 * half;
  float qx[NDB][16];
  float dot = 0.f;
  if constexpr (NORM) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 w = *(const u32x2*)((const bf16*)p.q + rowoff + 32 * db + 8 * i);
        qx[db][4 * i + 0] = __uint_as_float(w[0] << 16) * r_q;
        qx[db][4 * i + 1] = __uint_as_float(w[0] & 0xffff0000u) * r_q;
        qx[db][4 * i + 2] = __uint_as_float(w[1] << 16) * r_q;
        qx[db][4 * i + 3] = __uint_as_float(w[1] & 0xffff0000u) * r_q;
#pragma unroll
        for (int j = 0; j < 4; ++j) dot += dq[db][4 * i + j] * qx[db][4 * i + j];
      }
    dot = pair_sum(dot) * p.scale * (1.f / D);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gh = p.scale * dq[db][4 * i + j];
        v[j] = NORM ? r_q * (gh - qx[db][4 * i + j] * dot) : gh;
      }
      u32x2 w;
      w[0] = pack2(v[0], v[1]);
      w[1] = pack2(v[2], v[3]);
      *(u32x2*)((bf16*)p.dq + rowoff + 32 * db + 8 * i) = w;
    }
}

// ---------------------------------------------------------------- dK/dV kernel
template <int D, int BQ, bool NORM>
__global__ void __launch_bounds__(256, 1) attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = 4;
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;        // keys per workgroup
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per head row
  constexpr int NQC = BQ / 32;       // 32-row query chunks per block
  constexpr int QCPT = BQ * CPR / NT;  // Q_hat (and dO) chunks per thread per block
  static_assert((BK * CPR) % NT == 0 && (BQ * CPR) % NT == 0, "tiles must split evenly");
  static_assert(CPR == 16 || CPR == 8, "head_dim 64 or 128");

  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 dOs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dls[2][BQ];

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

  // ---- K_hat and V fragments (B operands of S = Q_hat K_hat^T and dP = dO V^T):
  // key l32 of this wave, head_dim 16kk + 8half + 0..7; rstd of this key.
  bf16x8 kf[KST], vf[KST];
  float r_k = 1.f;
  {
    const long first = ((long)b * T * p.Hkv + g) * D + (long)kb0 * kvstride;
    const uint32_t bytes = (uint32_t)max(0, T - kb0) * kvstride * 2;
    const auto rk = make_rsrc((const bf16*)p.k + first, bytes);
    const auto rv = make_rsrc((const bf16*)p.v + first, bytes);
    const uint32_t off = (uint32_t)((32 * wave + l32) * kvstride + 8 * half) * 2;
    float x[KST][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      unpack8(bload16(rk, off + 32 * kk), x[kk]);
      vf[kk] = __builtin_bit_cast(bf16x8, bload16(rv, off + 32 * kk));
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
    }
    if constexpr (NORM) r_k = fast_rsqrt(pair_sum(ss) * (1.f / D) + p.eps);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kk][e] *= r_k;
      kf[kk] = __builtin_bit_cast(bf16x8, pack8(x[kk]));
    }
  }

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
  int a_off[KST];  // 16-byte reads of Q_hat / dO rows 32qc + swap23(l32), chunk 2kk + half
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) a_off[kk] = swz_off<CPR>(swap23(l32), 16 * kk + 8 * half);
  int t_off[2][NDB];  // transpose reads of rows 32qc + 16ks + 8half + tq (+4), cols 32db + 16g1 + 4qq
  {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < NDB; ++db) t_off[hi][db] = swz_off<CPR>(8 * half + tq + 4 * hi, 32 * db + 16 * g1 + 4 * qq);
  }

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

  // ---- one step: S, dP, P, dS, dV, dK for this wave's 32 keys
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
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, pack8(ds + 8 * ks));
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
      }
    }
  };

  // one barrier per step: block it is read from one buffer while block it+1
  // (prefetched into registers when the step starts) is written to the other
  prefetch(0);
  stage(0);
  __syncthreads();
  auto step = [&](int buf, int it) {
    const bool more = it + 1 < nit;
    if (more) prefetch(it + 1);
    compute(buf, (qb_lo + it % nqb) * BQ);
    if (more) stage(buf ^ 1);
    __syncthreads();
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
  float dot = 0.f;
  float kx[NDB][16];
  if constexpr (NORM) {
    const bf16* kp = (const bf16*)p.k + ((long)b * T + key) * kvstride + (long)g * D + 4 * half;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 w = *(const u32x2*)(kp + 32 * db + 8 * i);
        kx[db][4 * i + 0] = __uint_as_float(w[0] << 16) * r_k;
        kx[db][4 * i + 1] = __uint_as_float(w[0] & 0xffff0000u) * r_k;
        kx[db][4 * i + 2] = __uint_as_float(w[1] << 16) * r_k;
        kx[db][4 * i + 3] = __uint_as_float(w[1] & 0xffff0000u) * r_k;
#pragma unroll
        for (int j = 0; j < 4; ++j) dot += dk_acc[db][4 * i + j] * kx[db][4 * i + j];
      }
    dot = pair_sum(dot) * p.scale * (1.f / D);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float dkv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g_hat = p.scale * dk_acc[db][4 * i + j];
        dkv[j] = NORM ? r_k * (g_hat - kx[db][4 * i + j] * dot) : g_hat;
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

template <int D>
static hipError_t launch_dkdv_d(const BwdParams& p, bool qk_norm, hipStream_t stream, const TimingEvents& kv_ev) {
  constexpr int BQ = 64;
  hipError_t e;
  const dim3 kgrid((unsigned)(p.nkb * p.B * p.Hkv));
  if (kv_ev.start != nullptr && (e = hipEventRecord(kv_ev.start, stream)) != hipSuccess) return e;
  if (qk_norm)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BQ, true>), kgrid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BQ, false>), kgrid, dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (kv_ev.stop != nullptr && (e = hipEventRecord(kv_ev.stop, stream)) != hipSuccess) return e;
  return hipSuccess;
}

template <int D, int HPW>
static hipError_t launch_bwd_d(const BwdParams& p, bool qk_norm, hipStream_t stream, const TimingEvents& dq_ev,
                               const TimingEvents& kv_ev) {
  constexpr int BN = 64;
  hipError_t e;
  const dim3 qgrid((unsigned)(p.nqb * p.B * p.Hkv * p.nsub));
  if (dq_ev.start != nullptr && (e = hipEventRecord(dq_ev.start, stream)) != hipSuccess) return e;
  if (qk_norm)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, BN, true>), qgrid, dim3(HPW * 256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, HPW, BN, false>), qgrid, dim3(HPW * 256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (dq_ev.stop != nullptr && (e = hipEventRecord(dq_ev.stop, stream)) != hipSuccess) return e;
  return launch_dkdv_d<D>(p, qk_norm, stream, kv_ev);
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int head_dim, bool qk_norm, hipStream_t stream,
                           const TimingEvents& kv_ev) {
  return head_dim == 128 ? launch_dkdv_d<128>(p, qk_norm, stream, kv_ev) : launch_dkdv_d<64>(p, qk_norm, stream, kv_ev);
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, int heads_per_wg, bool qk_norm, hipStream_t stream,
                      const TimingEvents& dq_ev, const TimingEvents& kv_ev) {
  if (head_dim == 128)
    return heads_per_wg == 2 ? launch_bwd_d<128, 2>(p, qk_norm, stream, dq_ev, kv_ev)
                             : launch_bwd_d<128, 1>(p, qk_norm, stream, dq_ev, kv_ev);
  return heads_per_wg == 2 ? launch_bwd_d<64, 2>(p, qk_norm, stream, dq_ev, kv_ev)
                           : launch_bwd_d<64, 1>(p, qk_norm, stream, dq_ev, kv_ev);
}

}  // namespace sa
