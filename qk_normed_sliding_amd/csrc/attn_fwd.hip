// Forward of QK-normed, grouped-query, sliding-window causal attention (gfx950).
//
// Computes, for every batch b and query head h (KV head g = h / G):
//   q_hat, k_hat = RMS-normed rows (no weight)        [post] QK-norm passage;
//                                                      [guide] 8.2.1 RMSNorm row
//   S_ij  = scale * <q_hat_i, k_hat_j> on the band 0 <= i - j <= W (W = -1: j <= i)
//                                                      [post] SSSL / sliding-window passage;
//                                                      [guide] 8.2.1 sliding-window row
//   O_i   = sum_j softmax_j(S_ij) v_j,  LSE_i = log sum_j exp(S_ij)
//
// Work decomposition (one workgroup = one 128-row query block of HPW query
// heads that share one KV head):
//   - 4 waves per head, 32 query rows per wave; the Q block is normalised in
//     registers once and kept there as the B operand of S^T = K_hat Q_hat^T.
//   - K/V tiles of BN keys are staged through LDS (double-buffered, global
//     loads of tile n+1 in flight while tile n is multiplied) and shared by
//     all heads of the workgroup; K rows are RMS-normed as they are staged.
//   - Only tiles that intersect the band are loaded; inside a tile each wave
//     skips 32-key chunks outside its own rows' band and masks only the
//     chunks that straddle the band edge.
//   - S^T puts one query row per lane (two lanes per row), so the row max and
//     sum need one lane-pair exchange. P leaves the accumulator already in
//     the K-slot order of the P.V MFMA; V is read K-major with the LDS
//     transpose read.
//   - With QK-norm the logits are bounded: |S| <= |scale| * D (the normed
//     rows have norm <= sqrt(D)). Then a fixed row maximum replaces the
//     running maximum (no rescaling of O, no max reduction): softmax is
//     invariant to the subtracted constant and exp stays in fp32/bf16 range
//     as long as 2 * |scale| * D stays well inside the exponent range, which
//     the host checks. Otherwise the running-maximum form is used.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

template <int D, int HPW, int BN, bool NORM, bool FIXED>
__global__ void __launch_bounds__(HPW * 4 * 64) attn_fwd_kernel(FwdParams p) {
  constexpr int WPH = 4;             // waves per head
  constexpr int BM = WPH * 32;       // query rows per block
  constexpr int NT = HPW * WPH * 64; // threads
  constexpr int KST = D / 16;        // MFMA k-steps over head_dim
  constexpr int NDB = D / 32;        // 32-wide head_dim blocks of O
  constexpr int LDP = D + 8;         // LDS row pitch in bf16 (16-byte pad)
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int CPT = BN * CPR / NT; // chunks per thread per tile
  constexpr int NCH = BN / 32;       // 32-key chunks per tile
  static_assert(CPT >= 1 && (BN * CPR) % NT == 0, "tile must split evenly over the threads");
  static_assert(!FIXED || NORM, "the fixed maximum needs normed rows");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * LDP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * LDP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Heavy query blocks first (the causal triangle makes late blocks longest).
  const int per_qb = p.B * p.Hkv * p.nsub;
  const int bid = blockIdx.x;
  const int qb = p.nqb - 1 - bid / per_qb;
  int rem = bid % per_qb;
  const int sub = rem % p.nsub;
  rem /= p.nsub;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const int head = g * p.G + sub * HPW + wave / WPH;
  const int r0 = qb * BM + (wave % WPH) * 32;  // first query row of this wave
  const int T = p.T;
  const int W = p.window;
  const long qstride = (long)p.Hq * D;
  const long kvstride = (long)p.Hkv * D;
  const bool wave_active = r0 < T;

  // ---- Q fragment: lane holds row r0 + l32, head_dim 16*kk + 8*half + 0..7.
  bf16x8 qf[KST];
  {
    const int row = r0 + l32;
    const bf16* src = (const bf16*)p.q + ((long)b * T + row) * qstride + (long)head * D + 8 * half;
    float x[KST][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < T) w = ld16(src + 16 * kk);
      unpack8(w, x[kk]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
    }
    float r = 1.f;
    if constexpr (NORM) r = fast_rsqrt(pair_sum(ss) * (1.f / D) + p.eps);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kk][e] *= r;
      qf[kk] = __builtin_bit_cast(bf16x8, pack8(x[kk]));
    }
  }

  // ---- key tiles that intersect the band of this block's rows
  const int row_lo = qb * BM;
  const int row_hi = min(T, row_lo + BM) - 1;
  const int key_lo = (W < 0) ? 0 : max(0, row_lo - W);
  const int n_lo = key_lo / BN;
  const int n_hi = row_hi / BN;

  const bf16* kbase = (const bf16*)p.k + (long)b * T * kvstride + (long)g * D;
  const bf16* vbase = (const bf16*)p.v + (long)b * T * kvstride + (long)g * D;

  u32x4 kreg[CPT], vreg[CPT];
  auto load_tile = [&](int n) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      const int key = n * BN + c / CPR;
      const int off = 8 * (c % CPR);
      u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
      if (key < T) {
        kz = ld16(kbase + key * kvstride + off);
        vz = ld16(vbase + key * kvstride + off);
      }
      kreg[i] = kz;
      vreg[i] = vz;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + NT * i;
      const int kt = c / CPR;
      const int off = 8 * (c % CPR);
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
      *(u32x4*)&Ks[buf][kt * LDP + off] = kw;
      *(u32x4*)&Vs[buf][kt * LDP + off] = vreg[i];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = FIXED ? p.c2 : -1e30f;  // base-2 row maximum
  float l_run = 0.f;                     // this lane's part of the row sum
  const int row = r0 + l32;

  load_tile(n_lo);
  for (int n = n_lo; n <= n_hi; ++n) {
    const int buf = (n - n_lo) & 1;
    store_tile(buf);
    __syncthreads();
    if (n < n_hi) load_tile(n + 1);
    if (!wave_active) continue;

    const bf16* Kb = Ks[buf];
    const bf16* Vb = Vs[buf];
    f32x16 s[NCH];
    bool act[NCH], edge[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int kc = n * BN + 32 * c;
      act[c] = !(kc > r0 + 31 || (W >= 0 && kc + 31 < r0 - W));
      edge[c] = !(kc + 31 <= r0 && (W < 0 || r0 + 31 - kc <= W));
      if (act[c]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[c][r] = 0.f;
        const bf16* kp = Kb + (32 * c + swap23(l32)) * LDP + 8 * half;
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) s[c] = mfma32(*(const bf16x8*)(kp + 16 * kk), qf[kk], s[c]);
      }
    }

    // logits -> base-2, mask on edge chunks
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (!act[c]) continue;
      const int kc = n * BN + 32 * c + 8 * half;
      if (edge[c]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kc + 16 * (r >> 3) + (r & 7);
          const bool ok = key <= row && (W < 0 || row - key <= W);
          s[c][r] = ok ? s[c][r] * p.c1 : -INFINITY;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[c][r] *= p.c1;
      }
    }

    float mref = m_run;
    if constexpr (!FIXED) {
      float mx = -1e30f;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (act[c])
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
      const float m_new = fmaxf(m_run, pair_max(mx));
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      mref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }

#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (!act[c]) continue;
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = fast_exp2(s[c][r] - mref);
        l_run += pv[r];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8(pv + 8 * ks));
        // V rows 32c + 16ks + 8*half + 0..7, read K-major with the transpose read
        const bf16* vp = Vb + (32 * c + 16 * ks + 8 * half + ((lane >> 2) & 3)) * LDP + 16 * ((lane >> 4) & 1) +
                         4 * (lane & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x4 lo = lds_read_tr(vp + 32 * db);
          const bf16x4 hi = lds_read_tr(vp + 32 * db + 4 * LDP);
          oacc[db] = mfma32(cat(lo, hi), pf, oacc[db]);
        }
      }
    }
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  if (row >= T) return;
  const float inv = 1.f / l_tot;
  bf16* dst = (bf16*)p.o + ((long)b * T + row) * qstride + (long)head * D + 4 * half;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack2(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv);
      w[1] = pack2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      *(u32x2*)(dst + 32 * db + 8 * i) = w;
    }
  if (half == 0) p.lse[((long)b * p.Hq + head) * T + row] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, int HPW>
static hipError_t launch_fwd_d(const FwdParams& p, bool qk_norm, bool fixed_max, hipStream_t stream,
                               const TimingEvents& ev) {
  constexpr int BN = 64;
  const dim3 grid((unsigned)(p.nqb * p.B * p.Hkv * p.nsub));
  const dim3 block(HPW * 4 * 64);
  if (ev.start != nullptr) {
    const hipError_t e = hipEventRecord(ev.start, stream);
    if (e != hipSuccess) return e;
  }
  if (qk_norm && fixed_max)
    hipLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, true, true>), grid, block, 0, stream, p);
  else if (qk_norm)
    hipLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, true, false>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, false, false>), grid, block, 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev.stop != nullptr) return hipEventRecord(ev.stop, stream);
  return e;
}

hipError_t launch_fwd(const FwdParams& p, int head_dim, int heads_per_wg, bool qk_norm, bool fixed_max,
                      hipStream_t stream, const TimingEvents& ev) {
  if (head_dim == 128)
    return heads_per_wg == 2 ? launch_fwd_d<128, 2>(p, qk_norm, fixed_max, stream, ev)
                             : launch_fwd_d<128, 1>(p, qk_norm, fixed_max, stream, ev);
  return heads_per_wg == 2 ? launch_fwd_d<64, 2>(p, qk_norm, fixed_max, stream, ev)
                           : launch_fwd_d<64, 1>(p, qk_norm, fixed_max, stream, ev);
}

}  // namespace sa
