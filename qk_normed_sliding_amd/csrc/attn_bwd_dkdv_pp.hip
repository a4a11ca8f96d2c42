// dK/dV kernel of the backward ([post] QK-norm and SSSL passages; [guide]
// 8.2.1), organised like the forward as two warp groups that take turns on the matrix cores. One
// workgroup owns 128 keys of one KV head (32 per wave of a group) and walks
// the query tiles (64 rows of one query head of the group) whose rows see
// them; the per-key state is split by role:
//   group A (waves 0-3) keeps k_hat and the dV accumulator:
//     M-phase of tile t: dV^T += dO^T P of tile t-1, S = Q_hat K_hat^T of tile t
//     V-phase of tile t: P = exp(S - LSE) (masked to the band), kept as the
//                        next dV operand and written to LDS for group B
//   group B (waves 4-7) keeps v and the dK accumulator:
//     M-phase of tile t: dK^T += Q_hat^T dS of tile t-1, dP = dO V^T of tile t
//     V-phase of tile t: dS = P (dP - Delta) with P from group A
// Group A runs M(t) in interval 2t and V(t) in 2t+1, group B one interval
// later, with a workgroup barrier between intervals: on every SIMD one wave
// works the matrix cores while its partner does the vector work. q_hat and
// dO tiles of 64 rows (plus their LSE and Delta) stream into three LDS slots
// as direct buffer-to-LDS copies; rows are XOR-swizzled so that the 16-byte
// row reads (S, dP) and the transpose reads (dV, dK) are bank-conflict free.
//
// The kernel is persistent: one workgroup per compute unit takes key blocks
// in a fixed heavy-first snake order (key blocks near the start of the
// sequence see the most query rows), or, in a launch of many rounds, a
// rotated order that runs a (batch, KV head)'s key blocks in the same round. At a block's end each wave issues the
// loads of its rows for the next block (k_hat or v) and that block's first
// tile before running the finished block's epilogue, so the epilogue, the
// next block's first loads and the workgroup's start overlap. The epilogue's
// RMS-norm backward takes k_hat from group A's operand registers (through
// LDS) and the row's 1/rms from the norm pass, so it reads no k row from
// memory.
#include "sa_common.h"
#include "sa_kernels.h"

#include <type_traits>

namespace sa {

// M-phase order for the scheduler: N1 operands of one 16-byte read each,
// then N2 operands of two transpose reads each, consumed in that order by one
// MFMA per operand, with the reads of operand i + LEAD issued after MFMA i.
template <int N1, int N2, int LEAD>
__device__ __forceinline__ void sched_mphase() {
  __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
  for (int i = 0; i < N1 - LEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < N2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
}

template <int D, bool ROPE, bool ROT>
__global__ void __launch_bounds__(512) attn_bwd_dkdv_pp_kernel(BwdParams p) {
  constexpr int NB = 3;
  constexpr int BQ = 64;               // query rows per tile (two 32-row chunks)
  constexpr int BK = 128;              // keys per workgroup (32 per wave of a group)
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TILE = BQ * D;
  constexpr int RPI = 64 / CPR;        // rows per direct-to-LDS instruction (1 KB)
  constexpr int IPW = BQ / RPI / 4;    // instructions per wave, per tile
  constexpr int LEAD = 4;              // operands in flight ahead of the MFMAs
  constexpr int kStoreOps = 32 / RPI;  // whole-row stores per wave of a finished block
  static_assert(KST == 2 * NDB, "operand groups of the row and transpose MFMAs have the same size");

  __shared__ __attribute__((aligned(1024))) bf16 Qs[NB][TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Os[NB][TILE];
  __shared__ __attribute__((aligned(1024))) bf16 Xs[4][2][2 * 512];  // P of a tile (2 chunks), per wave pair
  __shared__ __attribute__((aligned(16))) float Ls[NB][BQ];          // base-2 LSE of the tile's rows
  __shared__ __attribute__((aligned(16))) float Dl[NB][BQ];          // Delta of the tile's rows
  __shared__ __attribute__((aligned(1024))) bf16 Bs[4][32 * D];      // group B's per-key rows at a block change

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2;           // 0: S, P, dV   1: dP, dS, dK
  const int rw = wave & 3;             // 32-key slice
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = p.T;
  const int W = p.window;
  const uint32_t Wm = W < 0 ? 0x7fffffffu : (uint32_t)W;
  const int qstride = p.Hq * D;
  const int kvstride = p.Hkv * D;

  // ---- the workgroup's key blocks: ascending key blocks (the first see the
  // most queries), in a snake order over the workgroups (round k: item
  // k*G + w, or k*G + G-1-w on odd rounds)
  const int n_items = p.nkb * p.B * p.Hkv;
  const int NG = gridDim.x;
  auto item_index = [&](int k) { return k * NG + ((k & 1) ? NG - 1 - (int)blockIdx.x : (int)blockIdx.x); };
  // ROT (a problem of many rounds, at least two per key block: dkdv_rotated_order) takes them in a
  // rotated order instead: round k holds every key block of RC = NG / nkb (batch, KV head) pairs, and
  // workgroup w takes pair k RC + w mod RC, key block (w / RC + k) mod nkb. A pair's key blocks then
  // run together and share its q_hat / dO tiles in the caches (the heavy-first order visits them
  // rounds apart, which matters once a layer's rows outgrow the last-level cache), and every
  // workgroup cycles through all key blocks, so the rounds stay balanced.
  const int npair = p.B * p.Hkv;
  const int RC = ROT ? NG / p.nkb : 1;
  int n_blk = 0;
  if constexpr (ROT)
    n_blk = npair / RC;
  else
    while (item_index(n_blk) < n_items) ++n_blk;
  if (n_blk == 0) return;  // whole workgroup: no barrier has been passed

  // coordinates of the current block (set per block; the lambdas below read them)
  int kb = 0, g = 0, b = 0, kb0 = 0, kw0 = 0, key = 0, q_hi = 0, qb_lo = 0, nqb = 0, nit = 0;
  auto set_block = [&](int k) {
    int pair;
    if constexpr (ROT) {
      kb = ((int)blockIdx.x / RC + k) % p.nkb;
      pair = k * RC + (int)blockIdx.x % RC;
    } else {
      const int i = item_index(k);
      kb = i / npair;
      pair = i % npair;
    }
    g = pair / p.B;
    b = pair % p.B;
    kb0 = kb * BK;
    kw0 = kb0 + 32 * rw;  // first key of this wave
    key = kw0 + l32;
    // query blocks whose rows can see at least one key of this block
    q_hi = (W < 0) ? T - 1 : min(T - 1, kb0 + BK - 1 + W);
    qb_lo = kb0 / BQ;
    nqb = q_hi / BQ - qb_lo + 1;
    nit = p.G * nqb;  // tiles: (query head of the group, query block)
  };
  set_block(0);

  // ---- tile loads: instruction j of wave rw fills block m = 4j + rw, rows m*RPI + lane/CPR
  uint32_t ldo;
  {
    const int r = rw * RPI + lane / CPR;
    ldo = (uint32_t)((lane / CPR) * qstride + 8 * ((lane % CPR) ^ swz<CPR>(r))) * 2;
  }
  const uint32_t qs_lds = lds_addr(&Qs[0][0]);
  const uint32_t os_lds = lds_addr(&Os[0][0]);
  auto issue = [&](int it) __attribute__((always_inline)) {  // group A: q_hat rows and base-2 LSE; group B: dO rows and Delta
    const int hh = it / nqb;
    const int row0 = (qb_lo + it % nqb) * BQ;
    const int head = g * p.G + hh;
    const long first = ((long)b * T * p.Hq + head) * D;
    const u32x4 rs = rsrc_words((const bf16*)(grp == 0 ? p.qhat : p.dout) + first, (uint32_t)T * qstride * 2);
    const uint32_t slot = (grp == 0 ? qs_lds : os_lds) + (uint32_t)((it % NB) * TILE * 2);
    const uint32_t toff = (uint32_t)row0 * qstride * 2;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int m = 4 * j + rw;
      dma16(rs, uniform((int)(slot + m * 1024)), ldo + toff + (uint32_t)(m * RPI * qstride * 2), 0u);
    }
    if (rw == 0) {
      const float* src = (grp == 0 ? p.lse2 : p.delta) + ((long)b * p.Hq + head) * T;
      const u32x4 rl = rsrc_words(src, (uint32_t)T * 4);
      const uint32_t dst = lds_addr(grp == 0 ? &Ls[it % NB][0] : &Dl[it % NB][0]);
      dma4(rl, uniform((int)dst), (uint32_t)(row0 + lane) * 4);
    }
  };

  // ---- per-key fragments (B operands of S and dP): key l32, head_dim 16kk +
  // 8half. k_hat comes from the backward's norm pass (turned when rotary
  // tables are given), the same rows the dQ kernel's S uses.
  bf16x8 kf[KST];  // group A: k_hat;  group B: v
  auto load_kf = [&](bf16x8 (&dst)[KST]) __attribute__((always_inline)) {
    const long first = ((long)b * T * p.Hkv + g) * D + (long)kb0 * kvstride;
    const uint32_t bytes = (uint32_t)max(0, T - kb0) * kvstride * 2;
    const auto rk = make_rsrc((const bf16*)(grp == 0 ? p.khat : p.v) + first, bytes);
    const uint32_t off = (uint32_t)((32 * rw + l32) * kvstride + 8 * half) * 2;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) dst[kk] = __builtin_bit_cast(bf16x8, bload16(rk, off + 32 * kk));
  };
  load_kf(kf);

  // ---- per-key rows at a block change, through a per-wave staging area of 32
  // rows (group A: tile slots 1-2 of Os, which the next block does not load
  // before its first barrier; group B: Bs), row r's 16-byte chunk j at chunk
  // j ^ (r mod CPR), so that both directions are conflict free. The next
  // block's rows arrive by coalesced buffer-to-LDS copies (RPI whole rows per
  // instruction) and are read into the operand registers; the finished
  // block's dv or dk rows leave through the same area as whole rows. (The
  // lane index is made opaque where the addresses are formed, so that they
  // are computed at the block change, not kept in registers in between.)
  const uint32_t kst_lds = grp == 0 ? lds_addr(&Os[1][0]) + (uint32_t)(rw * 32 * D * 2) : lds_addr(&Bs[rw][0]);
  auto stage_rows = [&]() __attribute__((always_inline)) {
    int el = lane;
    asm volatile("" : "+v"(el));
    const long first = ((long)b * T * p.Hkv + g) * D + (long)kb0 * kvstride;
    const uint32_t bytes = (uint32_t)max(0, T - kb0) * kvstride * 2;
    const u32x4 rs = rsrc_words((const bf16*)(grp == 0 ? p.khat : p.v) + first, bytes);
#pragma unroll
    for (int m = 0; m < 32 / RPI; ++m) {
      const int r = m * RPI + el / CPR;  // row within the wave's 32 keys
      const int lc = (el % CPR) ^ (r % CPR);
      dma16(rs, uniform((int)(kst_lds + m * 1024)), (uint32_t)((32 * rw + r) * kvstride + 8 * lc) * 2, 0u);
    }
  };
  auto kf_from_stage = [&]() __attribute__((always_inline)) {
    int el = lane;
    asm volatile("" : "+v"(el));
    const int e32 = el & 31, eh = el >> 5;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      kf[kk] = *(SA_LDS const bf16x8*)(uintptr_t)(kst_lds + (uint32_t)(e32 * D * 2 + (((2 * kk + eh) ^ (e32 % CPR)) << 4)));
  };

  // ---- LDS read addresses (bytes): row reads of rows 32qc + swap23(l32),
  // head_dim 16kk + 8half: (slot + base) ^ (kk << 5); transpose reads of rows
  // 32qc + 16ks + 8half + tq (+4), columns 32db + 16g1 + 4qq: base ^ (db << 6).
  const uint32_t ra_base = (uint32_t)(swap23(l32) * D * 2 + (((half ^ swz<CPR>(swap23(l32))) & (CPR - 1)) << 4));
  uint32_t tr_base[2];
  {
    const int tq = (lane >> 2) & 3, g1 = (lane >> 4) & 1, qq = lane & 3;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) tr_base[hi] = (uint32_t)swz_off<CPR>(8 * half + tq + 4 * hi, 16 * g1 + 4 * qq) * 2;
  }
  auto lds_ld16 = [](uint32_t addr) { return *(SA_LDS const bf16x8*)(uintptr_t)addr; };
  auto lds_tr = [](uint32_t addr) { return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4*)(uintptr_t)addr); };
  // both chunks' rows, interleaved (chunk 0 k-step 0, chunk 1 k-step 0, ...),
  // the order in which the two S (or dP) chains consume them
  auto rows_load2 = [&](uint32_t slot, bf16x8 (&a0)[KST], bf16x8 (&a1)[KST]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      a0[kk] = lds_ld16(((slot + ra_base) ^ (uint32_t)(kk << 5)));
      a1[kk] = lds_ld16(((slot + ra_base) ^ (uint32_t)(kk << 5)) + 32 * D * 2);
    }
  };
  auto tr_load = [&](uint32_t slot, int qc, bf16x8 (&a)[KST]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t rb = slot + (uint32_t)((32 * qc + 16 * ks) * D * 2);
        a[ks * NDB + db] = cat(lds_tr(rb + (tr_base[0] ^ (uint32_t)(db << 6))), lds_tr(rb + (tr_base[1] ^ (uint32_t)(db << 6))));
      }
  };

  f32x16 acc[NDB];  // group A: dV^T, group B: dK^T (head_dim 32db + 8i + 4half + j, key l32)
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  f32x16 sc[2];     // S (A) or dP (B) of the current tile, from its M-phase to its V-phase
  bf16x8 op[2][2];  // P (A) or dS (B) of the previous tile: B operands of dV / dK

  // band test of chunk qc of tile it: register r of a lane holds query row
  // q0 + 16(r>>3) + 8half + (r&7) and key `key`. Rows past T need no mask:
  // their q_hat, dO, LSE and Delta arrive as zeros (the copies' range check),
  // so their finite P meets zero dO rows in dV and a zero dS in dK.
  auto chunk_q0 = [&](int it, int qc) { return (qb_lo + it % nqb) * BQ + 32 * qc; };
  auto chunk_edge = [&](int q0) {  // not every (row, key) pair of the chunk is inside the band
    return !(q0 >= kw0 + 31 && (W < 0 || q0 + 31 - kw0 <= W));
  };
  auto band_ok = [&](int q0, int r) {
    return (uint32_t)(q0 + 16 * (r >> 3) + 8 * half + (r & 7) - key) <= Wm;
  };
  auto xs_addr = [&](int qc, int ks) { return lds_addr(&Xs[rw][qc][ks * 512 + 8 * lane]); };

  // ---- M-phase of tile t (both groups): the row-operand chains of tile t
  // (A: S from q_hat rows, B: dP from dO rows; B operand kf), then the
  // transpose-operand MFMAs of tile t-1 (A: dV from dO^T and P, B: dK from
  // q_hat^T and dS). The first step has no tile t-1, the last no tile t.
  enum { K_FIRST = 0, K_MID = 1, K_LAST = 2 };
  auto m_phase = [&](int t, auto kind) __attribute__((always_inline)) {
    constexpr int K = decltype(kind)::value;
    constexpr bool CUR = K != K_LAST, PREV = K != K_FIRST;
    const uint32_t rows_slot = (grp == 0 ? qs_lds : os_lds) + (uint32_t)((t % NB) * TILE * 2);
    const uint32_t tr_slot = (grp == 0 ? os_lds : qs_lds) + (uint32_t)(((t + NB - 1) % NB) * TILE * 2);
    bf16x8 a0[KST], a1[KST], u0[KST], u1[KST];
    __builtin_amdgcn_s_setprio(1);
    if constexpr (CUR) rows_load2(rows_slot, a0, a1);
    if constexpr (PREV) {
      tr_load(tr_slot, 0, u0);
      tr_load(tr_slot, 1, u1);
    }
    if constexpr (CUR) {
      f32x16 c0 = mfma32(a0[0], kf[0], f32x16{});
      f32x16 c1 = mfma32(a1[0], kf[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < KST; ++kk) {
        c0 = mfma32(a0[kk], kf[kk], c0);
        c1 = mfma32(a1[kk], kf[kk], c1);
      }
      sc[0] = c0;
      sc[1] = c1;
    }
    if constexpr (PREV) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma32(u0[ks * NDB + db], op[0][ks], acc[db]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma32(u1[ks * NDB + db], op[1][ks], acc[db]);
    }
    if constexpr (CUR && PREV) sched_mphase<2 * KST, 2 * KST, LEAD>();
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- V-phase of tile t. A: P of tile t from S and the rows' LSE, masked
  // on chunks that cross the band edge; kept as the next dV operand and
  // written to LDS. B: dS of tile t = P (dP - Delta), P from LDS (written by A
  // one interval earlier).
  auto v_phase = [&](int t) __attribute__((always_inline)) {
    if (grp == 0) {
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const int q0 = chunk_q0(t, qc);
        const float* lse = &Ls[t % NB][32 * qc];
        float pr[16];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f32x4 l0 = *(const f32x4*)(lse + 16 * ks + 8 * half);
          const f32x4 l1 = *(const f32x4*)(lse + 16 * ks + 8 * half + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pr[8 * ks + e] = fast_exp2(__builtin_fmaf(sc[qc][8 * ks + e], p.c1, -(e < 4 ? l0[e] : l1[e - 4])));
        }
        if (chunk_edge(q0)) {  // one branch per chunk; the mask itself is a select per element
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = band_ok(q0, r) ? pr[r] : 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 w = pack8(pr + 8 * ks);
          op[qc][ks] = __builtin_bit_cast(bf16x8, w);
          *(SA_LDS u32x4*)(uintptr_t)xs_addr(qc, ks) = w;
        }
      }
    } else {
      const float* dl = &Dl[t % NB][0];
#pragma unroll
      for (int qc = 0; qc < 2; ++qc)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 w = *(SA_LDS const u32x4*)(uintptr_t)xs_addr(qc, ks);
          float pr[8];
          unpack8(w, pr);
          const f32x4 e0 = *(const f32x4*)(dl + 32 * qc + 16 * ks + 8 * half);
          const f32x4 e1 = *(const f32x4*)(dl + 32 * qc + 16 * ks + 8 * half + 4);
          float ds[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ds[e] = pr[e] * (sc[qc][8 * ks + e] - (e < 4 ? e0[e] : e1[e - 4]));
          op[qc][ks] = __builtin_bit_cast(bf16x8, pack8(ds));
        }
    }
  };

  // ---- schedule. Tile t is read in intervals 2t (A: q_hat rows), 2t+1 (A:
  // LSE; B: dO rows), 2t+2 (A: dO^T; B: Delta) and 2t+3 (B: q_hat^T). At the
  // start of its M-phase of tile s group A issues its half of tile s+1 (into
  // the slot of tile s-2, last read in interval 2s-1), and waits for it at the
  // end of its V-phase of tile s, before the barrier that publishes it. Group
  // B, whose matrix phase is the longer one, issues its half of tile s+2 at
  // the end of its V-phase of tile s instead (interval 2s+2, after the last
  // reads of the slot's tile s-1 in interval 2s), and waits for it a step
  // later; its half of tile 1 goes out with group A's at the start. Group A runs M(t) in interval 2t and V(t) in 2t+1, group B one
  // interval later; every wave passes 2*nit + 3 barriers (group B one at the
  // start, group A one after its last, empty, V-phase).
  // ---- the epilogue's k_hat exchange: group A wave rw leaves its k_hat
  // operands (lane l: key 32rw + l%32, head_dim 16kk + 8(l/32) .. +7) in LDS at
  // ((kk * 64 + l) * 16) bytes of a KST KB region shared with group B's wave rw
  // (the same keys), inside tile slots 1 and 2 of Qs, which the next block's
  // first load (slot 0) does not touch
  static_assert(4 * KST * 1024 <= 2 * TILE * 2, "the exchange fits in two tile slots");
  const uint32_t xk_lds = qs_lds + (uint32_t)(TILE * 2) + (uint32_t)(rw * KST * 1024);

  auto run = [&]() __attribute__((always_inline)) {
    if (1 < nit) issue(1);
    m_phase(0, std::integral_constant<int, K_FIRST>{});
    __syncthreads();
    v_phase(0);
    __builtin_amdgcn_s_waitcnt(0);
    if (grp == 1 && 2 < nit) issue(2);
    __syncthreads();
#pragma clang loop unroll(disable)
    for (int t = 1; t < nit; ++t) {
      if (grp == 0 && t + 1 < nit) issue(t + 1);
      m_phase(t, std::integral_constant<int, K_MID>{});
      __syncthreads();
      v_phase(t);
      __builtin_amdgcn_s_waitcnt(0);
      if (grp == 1 && t + 2 < nit) issue(t + 2);
      __syncthreads();
    }
    m_phase(nit, std::integral_constant<int, K_LAST>{});
    __syncthreads();
  };
  // 1/rms of this lane's key row (from the norm pass), one block ahead of its use
  const bool norm = p.qhat != p.q;
  auto load_rk = [&]() { return (grp == 1 && norm && key < T) ? p.rstd_k[((long)b * T + key) * p.Hkv + g] : 1.f; };
  float r_k = load_rk();
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int bk = 0; bk < n_blk; ++bk) {
    if (grp == 1) __syncthreads();
    run();
    if (grp == 0) __syncthreads();  // group A's last (empty) V-phase interval
    __builtin_amdgcn_s_waitcnt(0);
    // group A's k_hat rows for the epilogue's exchange, before the next block's rows replace them
    if (grp == 0 && norm) {
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        *(SA_LDS u32x4*)(uintptr_t)(xk_lds + (uint32_t)((kk * 64 + lane) * 16)) = __builtin_bit_cast(u32x4, kf[kk]);
    }
    // the finished block, for its epilogue; the next block's rows, 1/rms and first tile are loaded
    // meanwhile, and the epilogue's stores are issued after they have arrived, so that the wait
    // for them does not include the stores
    const int e_b = b, e_g = g, e_key = key, e_kw0 = kw0;
    const float e_rk = r_k;
    const bool more = bk + 1 < n_blk;
    if (more) {
      set_block(bk + 1);
      stage_rows();
      r_k = load_rk();
      issue(0);
    }
    __syncthreads();

    // ---- epilogue (the accumulators hold head_dim 32db + 8i + 4half + j of key `key`)
    if (grp == 1 && e_key < T) {
      // dk = r (dk_hat - k_hat <dk_hat, k_hat> / D), dk_hat = scale * acc, with
      // k_hat as the S MFMAs used it (bf16; with rotary tables the turned row,
      // and the result is turned back; head_dim d < D/2 in block db < NDB/2
      // pairs with d + D/2 in block db + NDB/2). Head_dim 32db + 8i + 4half + j
      // of the key sits in group A's operand kk = 2db + i/2 of lane
      // 32(i%2) + l%32, elements 4half + j.
      constexpr bool rope = ROPE;
      float dot = 0.f;
      u32x2 kh[NDB][4] = {};
      if (norm) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = 2 * db + i / 2, ln = 32 * (i % 2) + l32;
            kh[db][i] = *(SA_LDS const u32x2*)(uintptr_t)(xk_lds + (uint32_t)((kk * 64 + ln) * 16 + 8 * half));
            dot += acc[db][4 * i + 0] * __uint_as_float(kh[db][i][0] << 16);
            dot += acc[db][4 * i + 1] * __uint_as_float(kh[db][i][0] & 0xffff0000u);
            dot += acc[db][4 * i + 2] * __uint_as_float(kh[db][i][1] << 16);
            dot += acc[db][4 * i + 3] * __uint_as_float(kh[db][i][1] & 0xffff0000u);
          }
        dot = pair_sum(dot) * p.scale * (1.f / D);  // <dk_hat, k_hat> / D
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gh = p.scale * acc[db][4 * i + j];
            const uint32_t wd = kh[db][i][j >> 1];
            const float kx = __uint_as_float((j & 1) ? (wd & 0xffff0000u) : (wd << 16));
            acc[db][4 * i + j] = norm ? e_rk * (gh - kx * dot) : gh;
          }
      if (rope) {
        // the tables are read only now, when the k_hat words are dead: held across the
        // correction above they pushed the epilogue past the register file
        const long tr = (long)e_key * p.rope.stride + 4 * half;
        f32x4 tc[NDB / 2][4], ts[NDB / 2][4];
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            tc[db][i] = *(const f32x4*)(p.rope.cos + tr + 32 * db + 8 * i);
            ts[db][i] = *(const f32x4*)(p.rope.sin + tr + 32 * db + 8 * i);
          }
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 c = tc[db][i], sn = ts[db][i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float a = acc[db][4 * i + j], bb = acc[db + NDB / 2][4 * i + j];
              acc[db][4 * i + j] = a * c[j] + bb * sn[j];
              acc[db + NDB / 2][4 * i + j] = bb * c[j] - a * sn[j];
            }
          }
      }
    }
    // the rows and 1/rms of the next block have arrived (its first tile, issued last, may still
    // be in flight): the next rows go to the operand registers, then this block's dv (group A)
    // or dk (group B) rows leave through the staging area (a wave's LDS accesses stay in order,
    // so the reads see the rows first)
    if (more) {
      if (rw == 0)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW + 1) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
      kf_from_stage();
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    {
      int el = lane;
      asm volatile("" : "+v"(el));
      const int e32 = el & 31, eh = el >> 5;
      const uint32_t wbase = kst_lds + (uint32_t)(e32 * D * 2 + 8 * eh);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x2 w;
          w[0] = pack2(acc[db][4 * i], acc[db][4 * i + 1]);
          w[1] = pack2(acc[db][4 * i + 2], acc[db][4 * i + 3]);
          const int c = 4 * db + i;  // 16-byte chunk of head_dim 32db + 8i
          *(SA_LDS u32x2*)(uintptr_t)(wbase + (uint32_t)((c ^ (e32 % CPR)) << 4)) = w;
        }
      // (kStoreOps buffer stores per wave: rows at or past T fall outside the range, which ends
      // with head e_g's part of row T - 1, and are dropped)
      const auto rd = make_rsrc((bf16*)(grp == 0 ? p.dv : p.dk) + (long)e_b * T * kvstride + (long)e_g * D,
                                (uint32_t)(T * kvstride - e_g * D) * 2);
      const int crow = el / CPR, cch = el % CPR;
      u32x4 w[kStoreOps];  // all rows read before the first store: one LDS latency, not one per store
#pragma unroll
      for (int m = 0; m < kStoreOps; ++m) {
        const int r = RPI * m + crow;
        w[m] = *(SA_LDS const u32x4*)(uintptr_t)(kst_lds + (uint32_t)(r * D * 2 + ((cch ^ (r % CPR)) << 4)));
      }
      // the next block's first tile has landed before the stores are issued, which then stay in
      // flight across the barrier (the first vector phase's wait covers them). (A partial vmcnt
      // after the stores would not do: loads and stores are not retired in order with respect
      // to each other.) The rows are streamed past the L2 cache (non-temporal): nothing in this
      // pass reads them again, and the cache keeps serving the q_hat and dO tiles instead.
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int m = 0; m < kStoreOps; ++m)
        bstore16_nt(rd, (uint32_t)((e_kw0 + RPI * m + crow) * kvstride + 8 * cch) * 2, w[m]);
    }
    // the next block's accumulators start at zero
    if (more) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    }
    __syncthreads();
  }
}

// The rotated key-block order (see the kernel) for NG workgroups: RC = NG / nkb pairs per round, at
// least two rounds per key block.
bool dkdv_rotated_order(int NG, int nkb, int npair) {
  const int rc = NG % nkb == 0 ? NG / nkb : 0;
  return rc > 0 && npair % rc == 0 && npair / rc >= 2 * nkb;
}

template <int D, bool ROPE>
void launch_bwd_dkdv_pp_d(const BwdParams& p, dim3 grid, bool rot, hipStream_t stream, const TimingEvents& ev) {
  if (rot)
    hipExtLaunchKernelGGL((attn_bwd_dkdv_pp_kernel<D, ROPE, true>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
  else
    hipExtLaunchKernelGGL((attn_bwd_dkdv_pp_kernel<D, ROPE, false>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
}

hipError_t launch_bwd_dkdv_pp(const BwdParams& p, int head_dim, hipStream_t stream, const TimingEvents& ev) {
  const dim3 grid((unsigned)min(p.nkb * p.B * p.Hkv, p.nwg));
  const bool rot = dkdv_rotated_order((int)grid.x, p.nkb, p.B * p.Hkv);
  const bool rope = p.rope.cos != nullptr;
  if (head_dim == 128) {
    if (rope)
      launch_bwd_dkdv_pp_d<128, true>(p, grid, rot, stream, ev);
    else
      launch_bwd_dkdv_pp_d<128, false>(p, grid, rot, stream, ev);
  } else {
    if (rope)
      launch_bwd_dkdv_pp_d<64, true>(p, grid, rot, stream, ev);
    else
      launch_bwd_dkdv_pp_d<64, false>(p, grid, rot, stream, ev);
  }
  return hipGetLastError();
}

}  // namespace sa
