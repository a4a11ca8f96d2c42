// Forward of QK-normed, grouped-query, sliding-window causal attention for
// the main shape class: an even number of query heads per KV head, bounded
// logits (fixed row maximum), head_dim 64 or 128. Same computation as
// attn_fwd.hip ([post] QK-norm and SSSL passages; [guide] 8.2.1), organised
// for gfx950 as two warp groups that take turns on the matrix cores:
//
//   - One workgroup = one 128-row query block of 2 query heads sharing a KV
//     head; waves 0-3 (group 0) own the first head's rows, waves 4-7 (group
//     1) the second's, 32 rows per wave, q_hat normed in registers.
//   - A prologue kernel has written k_hat (normed key rows) and v_t (value
//     rows transposed to [D, keys]), so both tiles of 64 keys are plain
//     copies, issued as buffer loads straight into LDS (no registers, no
//     VALU) and XOR-swizzled so that the 16-byte operand reads of S = K Q^T
//     and of O^T += V^T P^T are bank-conflict free. Three buffers per operand
//     let the loads run two phases ahead of their use.
//   - Work per wave is split into an M-phase (the P.V MFMAs of the previous
//     tile plus the S MFMAs of the current one, with the LDS reads of the
//     next MFMA group in flight behind the current group) and a V-phase (the
//     exponentials and row sums of the current tile, then the next loads).
//     Group 1 runs one phase behind group 0 and the phases are separated by
//     workgroup barriers, so on every SIMD one wave is in its M-phase while
//     its partner is in its V-phase: matrix cores and vector ALUs overlap.
#include "sa_common.h"
#include "sa_kernels.h"

#include <type_traits>

namespace sa {

// Instruction order of an M-phase for the scheduler: the first operand
// group's LDS reads, then NPAIR groups in which every MFMA is followed by one
// read of the next group, then the last group's MFMAs. Each read so has a
// whole group of MFMAs (KST x 32 cycles) to land before it is used.
template <int KST, int NPAIR>
__device__ __forceinline__ void sched_pairs() {
  __builtin_amdgcn_sched_group_barrier(0x100, KST, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < NPAIR * KST; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, KST, 0);
}

// One 128-row query block of two query heads (the work of one workgroup).
// Ks and Vt are the LDS tile slots.
template <int D, int NB>
__device__ __forceinline__ void fwd_pp_block(const FwdParams& p, const int bid, bf16 (*Ks)[D * 64],
                                             bf16 (*Vt)[D * 64]) {
  constexpr int BN = 64;              // keys per tile
  constexpr int BM = 128;             // query rows per block (per head)
  constexpr int KST = D / 16;         // MFMA k-steps over head_dim = operand registers per 32-key chunk
  constexpr int NDB = D / 32;         // 32-wide head_dim blocks of O
  constexpr int CPR = D / 8;          // 16-byte chunks per K row
  constexpr int TILE = BN * D;        // elements of a K tile [64][D] or a V^T tile [D][64]
  constexpr int KRPI = 64 / CPR;      // K rows per direct-to-LDS instruction (1 KB)
  constexpr int KIPW = BN / KRPI / 4; // K instructions per wave of the loading group, per tile
  constexpr int VIPW = D / 8 / 4;     // V^T instructions per wave (8 rows of 128 B each)
  static_assert(KST == 2 * NDB, "one operand register set serves S and P.V chunks");
  static_assert(KIPW >= 1 && VIPW >= 1, "tile rows must split over the 4 waves of a group");
  static_assert(NB >= 3, "loads run two phases ahead of their first use");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2;           // warp group = query head within the pair
  const int rw = wave & 3;             // 32-row slice of the block
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Heavy query blocks first (the causal triangle makes late blocks longest).
  const int per_qb = p.B * p.Hkv * p.nsub;
  const int qb = p.nqb - 1 - bid / per_qb;
  int rem = bid % per_qb;
  const int sub = rem % p.nsub;
  rem /= p.nsub;
  const int g = rem % p.Hkv;
  const int b = rem / p.Hkv;
  const int head = g * p.G + sub * 2 + grp;
  const int r0 = qb * BM + rw * 32;    // first query row of this wave
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;
  const bool wave_active = r0 < T;
  const int row = r0 + l32;

  bf16x8 qf[KST];  // q_hat rows (B operand of S), filled below

  // ---- key tiles that intersect the band of this block's rows
  const int row_lo = qb * BM;
  const int row_hi = min(T, row_lo + BM) - 1;
  const int key_lo = (W < 0) ? 0 : max(0, row_lo - W);
  const int n_lo = key_lo / BN;
  const int ntile = row_hi / BN - n_lo + 1;

  // ---- direct-to-LDS loads. Instruction j of wave rw fills the 1 KB block
  // m = 4j + rw of the tile: K rows m*KRPI + lane/CPR, V^T rows 8m + lane/8.
  // The lane's physical chunk holds logical chunk (physical ^ swizzle(row));
  // with this block order the swizzle depends on rw and the lane only, so a
  // lane's offset is one per-lane base plus a uniform part. The whole offset
  // goes in the per-lane operand: the buffer's range check (rows past T read
  // as zero) covers that operand only.
  const u32x4 rk = rsrc_words((const bf16*)p.khat + ((long)b * T * p.Hkv + g) * D, (uint32_t)T * kvstride * 2);
  const u32x4 rv = rsrc_words((const bf16*)p.vt + ((long)b * p.Hkv + g) * D * p.Tp, (uint32_t)D * p.Tp * 2);
  uint32_t kdo, vdo;
  {
    const int r = rw * KRPI + lane / CPR;  // row of block m = rw (same swizzle as every m = 4j + rw)
    kdo = (uint32_t)((lane / CPR) * kvstride + 8 * ((lane % CPR) ^ swz<CPR>(r))) * 2;
    const int d = 8 * rw + lane / 8;
    vdo = (uint32_t)((lane / 8) * p.Tp + 8 * ((lane & 7) ^ swz<8>(d))) * 2;
  }
  const uint32_t ks_lds = lds_addr(&Ks[0][0]);
  const uint32_t vt_lds = lds_addr(&Vt[0][0]);
  auto issue_k = [&](int tau) {
    const uint32_t toff = (uint32_t)((n_lo + tau) * BN) * kvstride * 2;
    const uint32_t base = ks_lds + (uint32_t)((tau % NB) * TILE * 2);
#pragma unroll
    for (int j = 0; j < KIPW; ++j) {
      const int m = 4 * j + rw;
      dma16(rk, uniform((int)(base + m * 1024)), kdo + toff + (uint32_t)(m * KRPI * kvstride * 2), 0u);
    }
  };
  auto issue_v = [&](int tau) {
    const uint32_t toff = (uint32_t)((n_lo + tau) * BN) * 2;
    const uint32_t base = vt_lds + (uint32_t)((tau % NB) * TILE * 2);
#pragma unroll
    for (int j = 0; j < VIPW; ++j) {
      const int m = 4 * j + rw;
      dma16(rv, uniform((int)(base + m * 1024)), vdo + toff + (uint32_t)(m * 8 * p.Tp * 2), 0u);
    }
  };

  // ---- LDS operand reads (16 bytes each). Tile slots are 16 KB aligned and
  // the swizzle only flips byte-offset bits 4..7, so each read address is
  // (slot + lane base) ^ constant.
  // K: row 32c + swap23(l32), head_dim 16kk + 8half -> chunk (2kk + half) ^ swz(row)
  const uint32_t ka_base = (uint32_t)(swap23(l32) * D * 2 + (((half ^ swz<CPR>(swap23(l32))) & (CPR - 1)) << 4));
  // V^T: row l32 (+32db), keys 32c + 16ks + 8half -> chunk (4c + 2ks + half) ^ swz8(row)
  const uint32_t va_base = (uint32_t)(l32 * 128 + ((half ^ swz<8>(l32)) << 4));
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float l_run = 0.f;
  f32x16 s[2];          // logits of the tile between its M- and V-phase
  bf16x8 pf[2][2];      // probabilities of the previous tile (P.V operand)

  auto chunk_edge = [&](int t, int c) {  // not every (row, key) of the chunk is inside the band
    const int kc = t * BN + 32 * c;
    return !(kc + 31 <= r0 && (W < 0 || r0 + 31 - kc <= W));
  };

  // operand groups of one 32-key chunk: P.V (A = V^T rows, B = P^T) and S (A = K rows, B = Q^T)
  auto lds_ld16 = [](uint32_t addr) { return *(SA_LDS const bf16x8*)(uintptr_t)addr; };
  auto pv_load = [&](uint32_t vslot, int c, bf16x8 (&a)[KST]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t ad = (vslot + va_base) ^ (uint32_t)((4 * c + 2 * ks) << 4);
#pragma unroll
      for (int db = 0; db < NDB; ++db) a[ks * NDB + db] = lds_ld16(ad + db * 32 * 128);
    }
  };
  auto pv_mfma = [&](int c, const bf16x8 (&a)[KST]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(a[ks * NDB + db], pf[c][ks], oacc[db]);
  };
  auto s_load = [&](uint32_t kslot, int c, bf16x8 (&a)[KST]) {
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) a[kk] = lds_ld16(((kslot + ka_base) ^ (uint32_t)(kk << 5)) + c * 32 * D * 2);
  };
  auto s_mfma = [&](int c, const bf16x8 (&a)[KST]) {
    f32x16 acc = mfma32(a[0], qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < KST; ++kk) acc = mfma32(a[kk], qf[kk], acc);
    s[c] = acc;
  };

  // Tiles of the block that hold keys visible to some row of this wave.
  const int ta = (W < 0 ? 0 : max(0, r0 - W) / BN) - n_lo;
  const int tb = min(r0 + 31, row_hi) / BN - n_lo;

  // M-phase of tile tau: P.V of tile tau-1, then S of tile tau, each over
  // both 32-key chunks without masking (the V-phase zeroes probabilities of
  // keys outside the band). Straight-line: the reads of each operand group
  // are issued before the MFMAs of the group ahead of it. The first tile of
  // the wave has no P.V, the step after its last tile no S.
  enum { M_SKIP = 0, M_S = 1, M_FULL = 2, M_PV = 3 };
  auto m_phase = [&](int tau, auto kind) {
    constexpr int K = decltype(kind)::value;
    const uint32_t Vb = vt_lds + (uint32_t)(((tau + NB - 1) % NB) * TILE * 2);
    const uint32_t Kb = ks_lds + (uint32_t)((tau % NB) * TILE * 2);
    bf16x8 a0[KST], a1[KST];
    if constexpr (K == M_S) {
      s_load(Kb, 0, a0);
      s_load(Kb, 1, a1);
      s_mfma(0, a0);
      s_mfma(1, a1);
      sched_pairs<KST, 1>();
    } else if constexpr (K == M_PV) {
      pv_load(Vb, 0, a0);
      pv_load(Vb, 1, a1);
      pv_mfma(0, a0);
      pv_mfma(1, a1);
      sched_pairs<KST, 1>();
    } else if constexpr (K == M_FULL) {
      pv_load(Vb, 0, a0);
      pv_load(Vb, 1, a1);
      pv_mfma(0, a0);
      s_load(Kb, 0, a0);
      pv_mfma(1, a1);
      s_load(Kb, 1, a1);
      s_mfma(0, a0);
      s_mfma(1, a1);
      sched_pairs<KST, 3>();
    }
  };

  // V-phase of tile tau: probabilities against the fixed row maximum c2 (the
  // logits are bounded by |scale| * D), their bf16 operands and row sums.
  // Subtracting the bound keeps every probability <= 1, which measurably
  // improves the accuracy of the bf16 P.V products over leaving them
  // unshifted, even though both stay inside the fp32 range.
  auto v_phase = [&](int tau) {
    const int t = n_lo + tau;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float pv[16];
      if (chunk_edge(t, c)) {  // crosses the diagonal or the window start, or lies outside the band
        const uint32_t rk0 = (uint32_t)(row - (t * BN + 32 * c + 8 * half));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool ok = rk0 - (uint32_t)(16 * (r >> 3) + (r & 7)) <= Wm;
          pv[r] = ok ? fast_exp2(__builtin_fmaf(s[c][r], p.c1, -p.c2)) : 0.f;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(__builtin_fmaf(s[c][r], p.c1, -p.c2));
      }
      pf[c][0] = __builtin_bit_cast(bf16x8, pack8(pv));
      pf[c][1] = __builtin_bit_cast(bf16x8, pack8(pv + 8));
      float part[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) part[k] = (pv[4 * k] + pv[4 * k + 1]) + (pv[4 * k + 2] + pv[4 * k + 3]);
      l_run += (part[0] + part[1]) + (part[2] + part[3]);
    }
  };

  // ---- prologue loads: K tiles 0..NB-1 by group 1, V tiles 0..NB-2 by group 0
  if (grp == 1) {
    for (int tau = 0; tau < NB && tau < ntile; ++tau) issue_k(tau);
  } else {
    for (int tau = 0; tau < NB - 1 && tau < ntile; ++tau) issue_v(tau);
  }
  // ---- Q fragment (loaded while the first tiles are in flight): lane holds
  // row r0 + l32, head_dim 16*kk + 8*half + 0..7, normed.
  {
    const bf16* qbase = (const bf16*)p.q + ((long)b * T * p.Hq + head) * D;
    const auto rq = make_rsrc(qbase, (uint32_t)T * qstride * 2);
    const uint32_t off = (uint32_t)(row * qstride + 8 * half) * 2;
    float x[KST][8];
    float ss = 0.f;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      unpack8(bload16(rq, off + 32 * kk), x[kk]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[kk][e] * x[kk][e];
    }
    const float r = fast_rsqrt(pair_sum(ss) * (1.f / D) + p.eps);
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[kk][e] *= r;
      qf[kk] = __builtin_bit_cast(bf16x8, pack8(x[kk]));
    }
  }

  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed in LDS
  __syncthreads();

  // ---- phases. Group 0 runs M(tau) in interval 2tau and V(tau) in 2tau+1;
  // group 1 runs one interval later. Every wave passes the same 2*ntile + 2
  // barriers. In each V-phase the loading group first waits for the loads it
  // issued two intervals earlier (the barrier after it publishes them), then
  // issues the next: group 1 the K tile NB ahead of the tile it just
  // finished, group 0 the V tile NB-2 ahead. A K tile is read in the two
  // M-phases of its own tile, a V tile in the two that follow, and a slot is
  // refilled only after both, so no slot is overwritten while read.
  // The wave's own work covers tiles ta..tb; the steps before, at ta, inside,
  // at tb+1 and after run as separate loops, so that each loop body is
  // straight-line in the accumulators.
  auto step = [&](int tau, auto kind) {
    constexpr int K = decltype(kind)::value;
    if constexpr (K != M_SKIP) {
      __builtin_amdgcn_s_setprio(1);
      m_phase(tau, kind);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (grp == 1 && tau == ntile) return;  // group 1 ends on its last M-phase
    if constexpr (K == M_S || K == M_FULL) v_phase(tau);
    __builtin_amdgcn_s_waitcnt(0);
    if (grp == 0) {
      if (tau >= 1 && tau + NB - 2 < ntile) issue_v(tau + NB - 2);
    } else {
      if (tau + NB < ntile) issue_k(tau + NB);
    }
    __syncthreads();
  };
  using skip_t = std::integral_constant<int, M_SKIP>;
  if (grp == 1) __syncthreads();
  const int t_first = wave_active ? ta : ntile + 1;  // idle waves only pass barriers
  int tau = 0;
#pragma clang loop unroll(disable)
  for (; tau < t_first; ++tau) step(tau, skip_t{});
  if (wave_active) {
    step(tau++, std::integral_constant<int, M_S>{});
#pragma clang loop unroll(disable)
    for (; tau <= tb; ++tau) step(tau, std::integral_constant<int, M_FULL>{});
    step(tau++, std::integral_constant<int, M_PV>{});
#pragma clang loop unroll(disable)
    for (; tau <= ntile; ++tau) step(tau, skip_t{});
  }
  __builtin_amdgcn_s_waitcnt(0);

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
  if (half == 0) p.lse[((long)b * p.Hq + head) * T + row] = (p.c2 + fast_log2(l_tot)) * kLn2;
}

template <int D, int NB>
__global__ void __launch_bounds__(512) attn_fwd_pp_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) bf16 Ks[NB][D * 64];
  __shared__ __attribute__((aligned(1024))) bf16 Vt[NB][D * 64];
  fwd_pp_block<D, NB>(p, blockIdx.x, Ks, Vt);
}

hipError_t launch_fwd_pp(const FwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev) {
  constexpr int NB = 3;
  const dim3 grid((unsigned)(p.nqb * p.B * p.Hkv * p.nsub));
  if (ev.start != nullptr) {
    const hipError_t e = hipEventRecord(ev.start, stream);
    if (e != hipSuccess) return e;
  }
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_fwd_pp_kernel<128, NB>), grid, dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_pp_kernel<64, NB>), grid, dim3(512), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev.stop != nullptr) return hipEventRecord(ev.stop, stream);
  return e;
}

}  // namespace sa
