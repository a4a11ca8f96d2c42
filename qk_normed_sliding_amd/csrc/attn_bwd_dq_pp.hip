// dQ kernel of the backward, organised like attn_fwd_pp.hip: two warp groups
// (32 query rows per wave; the groups take two query heads of a KV group, or
// with an odd ratio alternate 32-row slices of 256 rows of one head)
// alternate M-phases and V-phases between workgroup barriers, and the key and
// value tiles arrive as plain buffer-to-LDS copies (k_hat from a norm
// prologue, v as stored). The gradient of [post] QK-norm and SSSL passages,
// [guide] 8.2.1:
//   S = K_hat q_hat^T, dP = V dO^T        (one query row per lane)
//   P = exp(S - LSE), dS = P (dP - Delta)  (V-phase)
//   dq_hat^T += K_hat^T dS^T                (next M-phase; K_hat read K-major
//                                             by the LDS transpose read)
// A key tile is read in the M-phase of its own tile (S) and of the next one
// (dQ), so K uses four LDS slots and V three.
#include "sa_common.h"
#include "sa_kernels.h"

#include <type_traits>

namespace sa {

template <int KST, int NPAIR, int RPM>
__device__ __forceinline__ void sched_dq_group() {
  // NPAIR MFMAs, each followed by RPM LDS reads of an operand group further on
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
}

template <int D>
__global__ void __launch_bounds__(512) attn_bwd_dq_pp_kernel(BwdParams p) {
  constexpr int NBK = 4, NBV = 3;
  constexpr int BN = 64;
  constexpr int BM = 128;
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TILE = BN * D;
  constexpr int KRPI = 64 / CPR;       // rows per direct-to-LDS instruction (1 KB)
  constexpr int IPW = BN / KRPI / 4;   // instructions per loading wave, per tile
  static_assert(KST == 2 * NDB, "operand groups of S/dP and dQ chunks have the same size");

  __shared__ __attribute__((aligned(1024))) bf16 Ks[NBK][TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Vs[NBV][TILE];
  __shared__ __attribute__((aligned(1024))) bf16 St[6][32 * D];  // prologue staging of waves 0-5

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2;
  const int rw = wave & 3;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int per_qb = p.B * p.Hkv * p.nsub;
  const int bid = blockIdx.x;
  // heavy query blocks first; a problem of many rounds of nwg workgroups (at least two per query
  // block) runs in chunks of RC = nwg / nqb (batch, KV head, sub) units instead, heavy-first inside
  // a chunk, so that a unit's query blocks run together and share its K/V band in the caches (the
  // workgroups are dispatched as compute units free up, which keeps the rounds balanced)
  const int RC = p.nwg % p.nqb == 0 ? p.nwg / p.nqb : 0;
  const bool chunked = RC > 0 && per_qb % RC == 0 && per_qb / RC >= 2 * p.nqb;
  const int CW = chunked ? RC : per_qb;
  const int qb = p.nqb - 1 - (bid % (CW * p.nqb)) / CW;
  int rem = (bid / (CW * p.nqb)) * CW + bid % CW;
  const int sub = rem % p.nsub;
  rem /= p.nsub;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  // rows of the block: the two groups take two query heads (same 128 rows),
  // or alternate 32-row slices of 256 rows of one head
  const int BMI = p.pair_rows ? 2 * BM : BM;
  const int head = g * p.G + (p.pair_rows ? sub : sub * 2 + grp);
  const int r0 = qb * BMI + (p.pair_rows ? 64 * rw + 32 * grp : 32 * rw);
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;
  const bool wave_active = r0 < T;
  const int row = r0 + l32;
  const bool norm = p.qhat != p.q;  // q_hat is written (and the norm backward applied) only with the QK-norm

  // ---- prologue: q_hat and dO fragments (B operands), r_q, Delta and LSE of
  // this lane's row. The q, dO and o rows of the wave are read with coalesced
  // 16-byte loads, QRPI whole rows per instruction (lane l: row QRPI*m +
  // l/CPR, chunk l%CPR); row sums of squares and of dO*o are reduced over
  // the CPR lanes of a row. q_hat is stored to the workspace from that same
  // layout, and q_hat and dO reach the MFMA operand layout (lane = row) through
  // a per-wave LDS staging area (row r's 16-byte chunk j at chunk j ^ (r mod
  // CPR): conflict-free in both directions). Waves 6 and 7 stage in K slot
  // NBK-1 and the per-row scalars go to V slot NBV-1; neither slot is loaded
  // before the first barrier.
  constexpr int QRPI = 64 / CPR;                // rows per coalesced instruction
  constexpr int QM = 32 / QRPI;                 // instructions per 32 rows
  const uint32_t stage = wave < 6 ? lds_addr(&St[wave][0]) : lds_addr(&Ks[NBK - 1][(wave - 6) * 32 * D]);
  float* scal = (float*)&Vs[NBV - 1][0] + wave * 64;  // [0, 32): r_q, [32, 64): Delta
  bf16x8 qf[KST], df[KST];
  float r_q = 1.f, delta = 0.f, lse2 = 0.f;

  // ---- key tiles that intersect the band of this block's rows
  const int row_lo = qb * BMI;
  const int row_hi = min(T, row_lo + BMI) - 1;
  const int key_lo = (W < 0) ? 0 : max(0, row_lo - W);
  const int n_lo = key_lo / BN;
  const int ntile = row_hi / BN - n_lo + 1;

  // ---- direct-to-LDS loads (same row layout for K_hat and V): instruction j
  // of wave rw fills the 1 KB block m = 4j + rw of the tile, rows m*KRPI + lane/CPR.
  const long kvfirst = ((long)b * T * p.Hkv + g) * D;
  const u32x4 rk = rsrc_words((const bf16*)p.khat + kvfirst, (uint32_t)T * kvstride * 2);
  const u32x4 rv = rsrc_words((const bf16*)p.v + kvfirst, (uint32_t)T * kvstride * 2);
  uint32_t ldo;
  {
    const int r = rw * KRPI + lane / CPR;  // same swizzle as every block m = 4j + rw
    ldo = (uint32_t)((lane / CPR) * kvstride + 8 * ((lane % CPR) ^ swz<CPR>(r))) * 2;
  }
  const uint32_t ks_lds = lds_addr(&Ks[0][0]);
  const uint32_t vs_lds = lds_addr(&Vs[0][0]);
  auto issue = [&](u32x4 rs, uint32_t slot_lds, int tau) {
    const uint32_t toff = (uint32_t)((n_lo + tau) * BN) * kvstride * 2;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int m = 4 * j + rw;
      dma16(rs, uniform((int)(slot_lds + m * 1024)), ldo + toff + (uint32_t)(m * KRPI * kvstride * 2), 0u);
    }
  };
  auto issue_k = [&](int tau) { issue(rk, ks_lds + (uint32_t)((tau % NBK) * TILE * 2), tau); };
  auto issue_v = [&](int tau) { issue(rv, vs_lds + (uint32_t)((tau % NBV) * TILE * 2), tau); };

  // ---- LDS operand reads. Rows 32c + swap23(l32), head_dim 16kk + 8half
  // (16-byte reads; address = (slot + base) ^ (kk << 5)), and the transpose
  // reads of K_hat rows 32c + 16ks + 8half + tq (+4), columns 32db + 16g1 + 4qq.
  const uint32_t ra_base = (uint32_t)(swap23(l32) * D * 2 + (((half ^ swz<CPR>(swap23(l32))) & (CPR - 1)) << 4));
  // (For another db only chunk bits 2.. change, and the swizzle XORs them, so the
  // address of block db is that of block 0 XOR (db << 6).)
  uint32_t kt_base[2];
  {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) kt_base[hi] = (uint32_t)swz_off<CPR>(8 * half + tq + 4 * hi, 16 * g1 + 4 * qq) * 2;
  }
  auto lds_ld16 = [](uint32_t addr) { return *(SA_LDS const bf16x8*)(uintptr_t)addr; };
  auto lds_tr = [](uint32_t addr) { return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4*)(uintptr_t)addr); };

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  f32x16 s[2], dp[2];   // S and dP of the tile between its M- and V-phase
  bf16x8 dsf[2][2];     // dS of the previous tile (B operand of the dQ MFMAs)

  auto rows_load = [&](uint32_t slot, int c, bf16x8 (&a)[KST]) {
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) a[kk] = lds_ld16(((slot + ra_base) ^ (uint32_t)(kk << 5)) + c * 32 * D * 2);
  };
  auto dq_load = [&](uint32_t slot, int c, bf16x8 (&a)[KST]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t rb = slot + (uint32_t)((32 * c + 16 * ks) * D * 2);
        a[ks * NDB + db] = cat(lds_tr(rb + (kt_base[0] ^ (uint32_t)(db << 6))), lds_tr(rb + (kt_base[1] ^ (uint32_t)(db << 6))));
      }
  };
  auto chain = [&](const bf16x8 (&a)[KST], const bf16x8 (&bv)[KST]) {
    f32x16 acc = mfma32(a[0], bv[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < KST; ++kk) acc = mfma32(a[kk], bv[kk], acc);
    return acc;
  };
  auto dq_mfma = [&](int c, const bf16x8 (&a)[KST]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = mfma32(a[ks * NDB + db], dsf[c][ks], dq[db]);
  };

  // Tiles of the block that hold keys visible to some row of this wave.
  const int ta = (W < 0 ? 0 : max(0, r0 - W) / BN) - n_lo;
  const int tb = min(r0 + 31, row_hi) / BN - n_lo;

  // M-phase of tile tau: dQ of tile tau-1, then S and dP of tile tau; the
  // operand reads of each group are in flight behind the MFMAs of the one
  // before (a window of KST reads).
  enum { M_SKIP = 0, M_SD = 1, M_FULL = 2, M_DQ = 3 };
  auto m_phase = [&](int tau, auto kind) {
    constexpr int K = decltype(kind)::value;
    const uint32_t Kp = ks_lds + (uint32_t)(((tau + NBK - 1) % NBK) * TILE * 2);
    const uint32_t Kc = ks_lds + (uint32_t)((tau % NBK) * TILE * 2);
    const uint32_t Vc = vs_lds + (uint32_t)((tau % NBV) * TILE * 2);
    bf16x8 a0[KST], a1[KST];
    if constexpr (K == M_DQ || K == M_FULL) {
      dq_load(Kp, 0, a0);
      dq_load(Kp, 1, a1);
      dq_mfma(0, a0);
      if constexpr (K == M_FULL) rows_load(Kc, 0, a0);
      dq_mfma(1, a1);
    }
    if constexpr (K == M_SD) rows_load(Kc, 0, a0);
    if constexpr (K == M_SD || K == M_FULL) {
      rows_load(Kc, 1, a1);
      s[0] = chain(a0, qf);
      rows_load(Vc, 0, a0);
      s[1] = chain(a1, qf);
      rows_load(Vc, 1, a1);
      dp[0] = chain(a0, df);
      dp[1] = chain(a1, df);
    }
    // Scheduling: MFMA i consumes operand i (a dQ operand is two transpose
    // reads, an S/dP operand one 16-byte read); the reads of operand i + LEAD
    // follow MFMA i, so LEAD operands are in flight.
    constexpr int LEAD = 3;
    if constexpr (K == M_FULL) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
#pragma unroll
      for (int i = 0; i < 2 * KST - LEAD; ++i) sched_dq_group<KST, 1, 2>();
#pragma unroll
      for (int i = 0; i < 4 * KST; ++i) sched_dq_group<KST, 1, 1>();
      __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
    } else if constexpr (K == M_SD) {
      __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
      for (int i = 0; i < 4 * KST - LEAD; ++i) sched_dq_group<KST, 1, 1>();
      __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
    } else if constexpr (K == M_DQ) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
#pragma unroll
      for (int i = 0; i < 2 * KST - LEAD; ++i) sched_dq_group<KST, 1, 2>();
      __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
    }
  };

  // V-phase of tile tau: P against the forward's LSE, dS, bf16 operands for dQ.
  // Register r of chunk c: key (n_lo+tau)*64 + 32c + 16(r>>3) + 8half + (r&7).
  auto chunk_edge = [&](int t, int c) {  // not every (row, key) of the chunk is inside the band
    const int kc = t * BN + 32 * c;
    return !(kc + 31 <= r0 && (W < 0 || r0 + 31 - kc <= W));
  };
  auto v_phase = [&](int tau) {
    const int t = n_lo + tau;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float ds[16];
      if (chunk_edge(t, c)) {
        const uint32_t rk0 = (uint32_t)(row - (t * BN + 32 * c + 8 * half));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = rk0 - (uint32_t)(16 * (r >> 3) + (r & 7)) <= Wm;
          const float pe = ok ? fast_exp2(__builtin_fmaf(s[c][r], p.c1, -lse2)) : 0.f;
          ds[r] = pe * (dp[c][r] - delta);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(s[c][r], p.c1, -lse2)) * (dp[c][r] - delta);
      }
      dsf[c][0] = __builtin_bit_cast(bf16x8, pack8(ds));
      dsf[c][1] = __builtin_bit_cast(bf16x8, pack8(ds + 8));
    }
  };

  // ---- prologue loads: this wave's rows first, then the first tiles (K
  // tiles 0..2 by group 1, V tiles 0..1 by group 0). Vector memory
  // operations retire in issue order, so the rows, issued first, can be
  // processed while the tiles are still arriving.
  const long lrow = ((long)b * p.Hq + head) * T + row;
  {
    const long first = ((long)b * T * p.Hq + head) * D;
    const uint32_t bytes = (uint32_t)T * qstride * 2;
    const auto rq = make_rsrc((const bf16*)p.q + first, bytes);
    const auto rd = make_rsrc((const bf16*)p.dout + first, bytes);
    const auto ro = make_rsrc((const bf16*)p.o + first, bytes);
    const int crow = lane / CPR, cch = lane % CPR;  // row within an instruction, chunk
    u32x4 xq[QM], xd[QM], xo[QM];
#pragma unroll
    for (int m = 0; m < QM; ++m) {
      const uint32_t off = (uint32_t)((r0 + QRPI * m + crow) * qstride + 8 * cch) * 2;
      xq[m] = bload16_nt(rq, off);  // q and o rows are read once in the backward;
      xd[m] = bload16(rd, off);     // dO rows again as the dK/dV kernel's tiles
      xo[m] = bload16_nt(ro, off);
    }
    if (grp == 1) {
      for (int tau = 0; tau < 3 && tau < ntile; ++tau) issue_k(tau);
    } else {
      for (int tau = 0; tau < 2 && tau < ntile; ++tau) issue_v(tau);
    }
    // rotary table entries of the lane's rows and dimensions, in flight with the rows
    const bool rope = p.rope.cos != nullptr;
    f32x4 tab[QM][4];  // cos (2 x 4), sin (2 x 4)
    if (rope) {
      const auto rc = make_rsrc(p.rope.cos, 0xffffffffu);
      const auto rs = make_rsrc(p.rope.sin, 0xffffffffu);
#pragma unroll
      for (int m = 0; m < QM; ++m) {
        const uint32_t off =
            (uint32_t)(min(r0 + QRPI * m + crow, T - 1) * p.rope.stride + 8 * (cch % (CPR / 2))) * 4;
        tab[m][0] = __builtin_bit_cast(f32x4, bload16(rc, off));
        tab[m][1] = __builtin_bit_cast(f32x4, bload16(rc, off + 16));
        tab[m][2] = __builtin_bit_cast(f32x4, bload16(rs, off));
        tab[m][3] = __builtin_bit_cast(f32x4, bload16(rs, off + 16));
      }
    }
#pragma unroll
    for (int m = 0; m < QM; ++m) {
      const int r = QRPI * m + crow;  // row within the wave's 32
      float f[8], dv[8], ov[8];
      unpack8(xq[m], f);
      unpack8(xd[m], dv);
      unpack8(xo[m], ov);
      float ss = 0.f, dd = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss += f[e] * f[e];
        dd += dv[e] * ov[e];
      }
      ss = group_sum<CPR>(ss);
      dd = group_sum<CPR>(dd);
      const float rr = norm ? fast_rsqrt(ss * (1.f / D) + p.eps) : 1.f;
      if (rope) {
        // the partner chunk (other half of the row) is CPR/2 lanes away:
        // lower half x c - x' s, upper half x c + x' s
        float fp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) fp[e] = __shfl_xor(f[e], CPR / 2);
        const float sg = cch >= CPR / 2 ? 1.f : -1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          f[e] = __builtin_fmaf(f[e], tab[m][e / 4][e % 4], sg * fp[e] * tab[m][2 + e / 4][e % 4]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= rr;
      const u32x4 w = pack8(f);
      const uint32_t at = stage + (uint32_t)(r * D * 2 + ((cch ^ (r % CPR)) << 4));
      *(SA_LDS u32x4*)(uintptr_t)at = norm ? w : xq[m];
      if (cch == 0) {
        scal[r] = rr;
        scal[32 + r] = dd;
      }
    }
    const float lse_raw = row < T ? p.lse[lrow] : 0.f;  // (its latency overlaps the staging below)
    // lane = row reads (the same wave wrote them; LDS keeps a wave's order)
    const uint32_t rbase = stage + (uint32_t)(l32 * D * 2);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qf[kk] = *(SA_LDS const bf16x8*)(uintptr_t)(rbase + (uint32_t)((((2 * kk + half) ^ (l32 % CPR))) << 4));
    r_q = scal[l32];
    delta = scal[32 + l32];
    lse2 = row < T ? lse_raw * kLog2e : INFINITY;
    // every load and tile copy of the prologue has landed before the first
    // store is issued: the stores below are then left in flight across the
    // barrier (the first vector phase's wait covers them). (A partial vmcnt
    // after the stores would not do: loads and stores are not retired in
    // order with respect to each other.)
    __builtin_amdgcn_s_waitcnt(0);
    if (half == 0 && row < T) {
      p.delta[lrow] = delta;
      p.lse2[lrow] = lse2;  // for the dK/dV kernel's probabilities
    }
    // the q_hat rows for the dK/dV kernel, read back from the staging area
    // (rows at or past T are dropped by the buffer's range)
    if (norm) {
      const auto rqh = make_rsrc((bf16*)p.qhat + first, bytes);
#pragma unroll
      for (int m = 0; m < QM; ++m) {
        const int r = QRPI * m + crow;
        const u32x4 w = *(SA_LDS const u32x4*)(uintptr_t)(stage + (uint32_t)(r * D * 2 + ((cch ^ (r % CPR)) << 4)));
        bstore16(rqh, (uint32_t)((r0 + r) * qstride + 8 * cch) * 2, w);
      }
    }
#pragma unroll
    for (int m = 0; m < QM; ++m) {
      const int r = QRPI * m + crow;
      *(SA_LDS u32x4*)(uintptr_t)(stage + (uint32_t)(r * D * 2 + ((cch ^ (r % CPR)) << 4))) = xd[m];
    }
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      df[kk] = *(SA_LDS const bf16x8*)(uintptr_t)(rbase + (uint32_t)((((2 * kk + half) ^ (l32 % CPR))) << 4));
  }
  __syncthreads();

  // ---- phases: group 0 runs M(tau) in interval 2tau and V(tau) in 2tau+1,
  // group 1 one interval later; every wave passes 2*ntile + 2 barriers. In
  // its V-phase a loading group waits for the loads it issued two intervals
  // earlier, then issues the next: group 1 the K tile 3 ahead of the tile it
  // finished (its slot held the tile read by both groups' M-phases up to the
  // interval before), group 0 the V tile 2 ahead.
  auto step = [&](int tau, auto kind) {
    constexpr int K = decltype(kind)::value;
    if constexpr (K != M_SKIP) {
      __builtin_amdgcn_s_setprio(1);
      m_phase(tau, kind);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (grp == 1 && tau == ntile) return;
    if constexpr (K == M_SD || K == M_FULL) v_phase(tau);
    __builtin_amdgcn_s_waitcnt(0);
    if (grp == 0) {
      if (tau + 2 < ntile) issue_v(tau + 2);
    } else {
      if (tau + 3 < ntile) issue_k(tau + 3);
    }
    __syncthreads();
  };
  using skip_t = std::integral_constant<int, M_SKIP>;
  if (grp == 1) __syncthreads();
  const int t_first = wave_active ? ta : ntile + 1;
  int tau = 0;
#pragma clang loop unroll(disable)
  for (; tau < t_first; ++tau) step(tau, skip_t{});
  if (wave_active) {
    step(tau++, std::integral_constant<int, M_SD>{});
#pragma clang loop unroll(disable)
    for (; tau <= tb; ++tau) step(tau, std::integral_constant<int, M_FULL>{});
    step(tau++, std::integral_constant<int, M_DQ>{});
#pragma clang loop unroll(disable)
    for (; tau <= ntile; ++tau) step(tau, skip_t{});
  }
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: dq = r (dq_hat - q_hat <dq_hat, q_hat> / D), dq_hat = scale * acc
  // (with rotary tables q_hat is the turned row and the result is turned back).
  // The accumulator holds head_dim 32db + 8i + 4half + j of this lane's row;
  // q_hat (bf16, as the S MFMAs used it) comes from the operand registers,
  // which hold head_dim 16kk + 8half + e. With i = 2a + c, the element sits in
  // register kk = 2db + a, element 4half + j, of lane half' = c: this lane's
  // own quad for c = half, the partner lane's (l ^ 32) for c != half. One
  // lane-pair swap per dword of (low quad, high quad) delivers, in the low
  // quad register, the elements for c = 0 and in the high quad register those
  // for c = 1, in both lane halves.
  // Lanes of rows past T compute on zero accumulators (their probabilities
  // were zero) and are not stored; they stay for the staged stores below.
  if (!wave_active) return;
  // rotary table entries of the row, loaded first (head_dim d < D/2 in block
  // db < NDB/2 pairs with d + D/2 in block db + NDB/2)
  const bool rope = p.rope.cos != nullptr;
  f32x4 tc[NDB / 2][4], ts[NDB / 2][4];
  if (rope) {
    const long tr = (long)min(row, T - 1) * p.rope.stride + 4 * half;
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tc[db][i] = *(const f32x4*)(p.rope.cos + tr + 32 * db + 8 * i);
        ts[db][i] = *(const f32x4*)(p.rope.sin + tr + 32 * db + 8 * i);
      }
  }
  float qx[NDB][16];
  float dot = 0.f;
  if (norm) {
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      const u32x4 w = __builtin_bit_cast(u32x4, qf[kk]);
      const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
      const int db = kk >> 1, a = kk & 1;
      // c = 0: i = 2a; c = 1: i = 2a + 1
      const uint32_t lo[2] = {(uint32_t)s0[0], (uint32_t)s1[0]};
      const uint32_t hi[2] = {(uint32_t)s0[1], (uint32_t)s1[1]};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        qx[db][4 * (2 * a) + 2 * t] = __uint_as_float(lo[t] << 16);
        qx[db][4 * (2 * a) + 2 * t + 1] = __uint_as_float(lo[t] & 0xffff0000u);
        qx[db][4 * (2 * a + 1) + 2 * t] = __uint_as_float(hi[t] << 16);
        qx[db][4 * (2 * a + 1) + 2 * t + 1] = __uint_as_float(hi[t] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dot += dq[db][r] * qx[db][r];
    dot = pair_sum(dot) * p.scale * (1.f / D);
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float gh = p.scale * dq[db][r];
      dq[db][r] = norm ? r_q * (gh - qx[db][r] * dot) : gh;
    }
  if (rope) {
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 c = tc[db][i], sn = ts[db][i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = dq[db][4 * i + j], bb = dq[db + NDB / 2][4 * i + j];
          dq[db][4 * i + j] = a * c[j] + bb * sn[j];
          dq[db + NDB / 2][4 * i + j] = bb * c[j] - a * sn[j];
        }
      }
  }
  // The wave's 32 rows go through its staging area (free again: every M-phase
  // ended before the last barrier), row r's 16-byte chunk j at chunk
  // j ^ (r mod CPR) as in the prologue, and leave as whole rows: each store
  // instruction writes QRPI rows of D contiguous values, streamed past the L2
  // cache (non-temporal), which keeps serving the K and V tiles instead. (The lane index is
  // made opaque so that these addresses are computed here, not kept in
  // registers from the prologue's equal ones.)
  int el = lane;
  asm volatile("" : "+v"(el));
  const int el32 = el & 31;
  const uint32_t wbase = stage + (uint32_t)(el32 * D * 2 + 8 * (el >> 5));
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack2(dq[db][4 * i], dq[db][4 * i + 1]);
      w[1] = pack2(dq[db][4 * i + 2], dq[db][4 * i + 3]);
      const int c = 4 * db + i;  // 16-byte chunk of head_dim 32db + 8i
      *(SA_LDS u32x2*)(uintptr_t)(wbase + (uint32_t)((c ^ (el32 % CPR)) << 4)) = w;
    }
  const int crow = el / CPR, cch = el % CPR;
  const long first = ((long)b * T * p.Hq + head) * D;
#pragma unroll
  for (int m = 0; m < QM; ++m) {
    const int r = QRPI * m + crow;  // row within the wave's 32
    const u32x4 w = *(SA_LDS const u32x4*)(uintptr_t)(stage + (uint32_t)(r * D * 2 + ((cch ^ (r % CPR)) << 4)));
    if (r0 + r < T) st16_nt((bf16*)p.dq + first + (long)(r0 + r) * qstride + 8 * cch, w);
  }
}

hipError_t launch_bwd_dq_pp(const BwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev) {
  const dim3 grid((unsigned)(p.nqb * p.B * p.Hkv * p.nsub));
  if (head_dim == 128)
    hipExtLaunchKernelGGL((attn_bwd_dq_pp_kernel<128>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((attn_bwd_dq_pp_kernel<64>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

}  // namespace sa
