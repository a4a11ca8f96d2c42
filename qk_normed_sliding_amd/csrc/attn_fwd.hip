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
//   - K/V tiles of BN keys are staged through LDS and shared by all heads of
//     the workgroup; K rows are RMS-normed as they are staged. Double
//     buffering with one barrier per tile: the buffer loads of tile n+1 are
//     issued when tile n starts and written to the other buffer while tile n
//     is multiplied.
//     K rows are padded to 272 bytes and V rows to 320 bytes, which makes the
//     K-operand 16-byte reads and the V transpose reads bank-conflict free.
//   - Only tiles that intersect the band are loaded; inside a tile each wave
//     skips 32-key chunks outside its own rows' band and masks only the
//     chunks that straddle the band edge (one unsigned compare per logit).
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
  constexpr int KP = D + 8;          // K row pitch (bf16): 16-byte reads of 16 rows hit 16 bank groups
  constexpr int VP = D + 32;         // V row pitch (bf16): 4 rows of a transpose read hit disjoint banks
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int CPT = BN * CPR / NT; // chunks per thread per tile
  constexpr int NCH = BN / 32;       // 32-key chunks per tile
  static_assert(CPT >= 1 && (BN * CPR) % NT == 0, "tile must split evenly over the threads");
  static_assert(!FIXED || NORM, "the fixed maximum needs normed rows");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * VP];

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
  const int r0 = qb * BM + (wave % WPH) * 32;  // first query row of this wave (wave-uniform)
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;  // band test: (unsigned)(i - j) <= Wm
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;
  const bool wave_active = r0 < T;

  // ---- Q fragment: lane holds row r0 + l32, head_dim 16*kk + 8*half + 0..7.
  bf16x8 qf[KST];
  {
    const bf16* qbase = (const bf16*)p.q + ((long)b * T * p.Hq + head) * D;
    const auto rq = make_rsrc(qbase, (uint32_t)T * qstride * 2);
    const uint32_t off = (uint32_t)((r0 + l32) * qstride + 8 * half) * 2;
    float x[KST][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      unpack8(bload16(rq, off + 32 * kk), x[kk]);
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

  const bf16* kbase = (const bf16*)p.k + ((long)b * T * p.Hkv + g) * D;
  const bf16* vbase = (const bf16*)p.v + ((long)b * T * p.Hkv + g) * D;
  uint32_t ld_off[CPT];   // byte offset of this thread's chunks inside a tile (global)
  int st_k[CPT], st_v[CPT];  // element offset of the same chunks inside the LDS tiles
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + NT * i;
    ld_off[i] = (uint32_t)((c / CPR) * kvstride + 8 * (c % CPR)) * 2;
    st_k[i] = (c / CPR) * KP + 8 * (c % CPR);
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

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = FIXED ? p.c2 : -1e30f;  // base-2 row maximum
  float l_run = 0.f;                     // this lane's part of the row sum
  const int row = r0 + l32;

  // lane parts of the LDS read addresses
  const int k_lane = swap23(l32) * KP + 8 * half;
  const int v_lane = (8 * half + ((lane >> 2) & 3)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // P.V for one 32-key chunk given its 16 probabilities (K-slot order)
  auto pv_chunk = [&](const bf16* Vb, int c, const float* pv) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pack8(pv + 8 * ks));
      // V rows 32c + 16ks + 8*half + 0..7, read K-major with the transpose read
      const bf16* vp = Vb + (32 * c + 16 * ks) * VP + v_lane;
      bf16x4 lo[NDB], hi[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        lo[db] = lds_read_tr(vp + 32 * db);
        hi[db] = lds_read_tr(vp + 32 * db + 4 * VP);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(cat(lo[db], hi[db]), pf, oacc[db]);
    }
  };
  auto s_chunk = [&](const bf16* Kb, int c) {
    const bf16* kp = Kb + 32 * c * KP + k_lane;
    bf16x8 ka[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) ka[kk] = *(const bf16x8*)(kp + 16 * kk);
    f32x16 acc = mfma32(ka[0], qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < KST; ++kk) acc = mfma32(ka[kk], qf[kk], acc);
    return acc;
  };

  // Interior tile (fixed maximum): every chunk is inside the band for every
  // wave, so no masks and no per-chunk branches. The next tile's LDS store is
  // placed between the chunks so its VALU/LDS work overlaps the MFMAs.
  auto tile_interior = [&](const bf16* Kb, const bf16* Vb, bf16* Kn, bf16* Vn, bool store_next) {
    f32x16 s[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) s[c] = s_chunk(Kb, c);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = fast_exp2(__builtin_fmaf(s[c][r], p.c1, -m_run));
        l_run += pv[r];
      }
      if (c == NCH - 1 && store_next) store_tile(Kn, Vn);
      pv_chunk(Vb, c, pv);
    }
  };

  // General tile: per-wave chunk skipping, masks on edge chunks, and the
  // running maximum when the logits are not bounded.
  auto tile_general = [&](const bf16* Kb, const bf16* Vb, int n) {
    f32x16 s[NCH];
    bool act[NCH], edge[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int kc = n * BN + 32 * c;
      act[c] = !(kc > r0 + 31 || (W >= 0 && kc + 31 < r0 - W));
      edge[c] = !(kc + 31 <= r0 && (W < 0 || r0 + 31 - kc <= W));
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (act[c]) s[c] = s_chunk(Kb, c);

    float mref = m_run;
    if constexpr (!FIXED) {
      float mx = -1e30f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!act[c]) continue;
        if (edge[c]) {
          const uint32_t rk = (uint32_t)(row - (n * BN + 32 * c + 8 * half));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = rk - (uint32_t)(16 * (r >> 3) + (r & 7)) <= Wm;
            s[c][r] = ok ? s[c][r] * p.c1 : -INFINITY;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[c][r] *= p.c1;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c][r]);
      }
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
      if constexpr (FIXED) {
        if (edge[c]) {
          const uint32_t rk = (uint32_t)(row - (n * BN + 32 * c + 8 * half));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool ok = rk - (uint32_t)(16 * (r >> 3) + (r & 7)) <= Wm;
            pv[r] = ok ? fast_exp2(__builtin_fmaf(s[c][r], p.c1, -mref)) : 0.f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(__builtin_fmaf(s[c][r], p.c1, -mref));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(s[c][r] - mref);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) l_run += pv[r];
      pv_chunk(Vb, c, pv);
    }
  };

  // A tile is interior for the whole block when all its keys are at or
  // before the block's first row and within the window of its last row.
  const bool block_full = row_lo + BM <= T;
  auto interior = [&](int n) {
    return FIXED && block_full && n * BN + BN - 1 <= row_lo && (W < 0 || row_hi - n * BN <= W);
  };
  // One barrier per tile: tile n is read from one buffer while tile n+1
  // (prefetched into registers at the start of the step) is written to the
  // other; the barrier at the end publishes it and retires the reads.
  auto step = [&](const bf16* Kb, const bf16* Vb, bf16* Kn, bf16* Vn, int n) {
    const bool more = n < n_hi;
    if (more) load_tile(n + 1);
    if (interior(n)) {
      tile_interior(Kb, Vb, Kn, Vn, more);
    } else {
      if (wave_active) tile_general(Kb, Vb, n);
      if (more) store_tile(Kn, Vn);
    }
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
  if (qk_norm && fixed_max)
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, true, true>), grid, block, 0, stream, ev.start, ev.stop, 0, p);
  else if (qk_norm)
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, true, false>), grid, block, 0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((attn_fwd_kernel<D, HPW, BN, false, false>), grid, block, 0, stream, ev.start, ev.stop, 0, p);
  return hipGetLastError();
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
