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
//   1. pre-pass: Delta = rowsum(dO * O) and zeroing of the fp32 dQ accumulator;
//   2. main: one workgroup per (batch, KV head, 128-key block); 4 waves own
//      32 keys each and keep K_hat, V and the dK/dV accumulators in registers
//      while streaming every (query head of the group, 64-row query block) of
//      the band through LDS. S and dP come out with one key per lane; P and
//      dS then feed dV^T += dO^T P and dK^T += Q_hat^T dS directly (operands
//      dO^T and Q_hat^T via the LDS transpose read). dS goes to LDS once and
//      the workgroup computes its dQ_hat contribution for all 128 keys,
//      added to the fp32 accumulator with hardware float atomics;
//   3. finalize: dq = norm-backward(dQ_hat) -> bf16.
#include "sa_common.h"
#include "sa_kernels.h"

namespace sa {

// ---------------------------------------------------------------- pre-pass
template <int D>
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
__global__ void __launch_bounds__(256) attn_bwd_kernel(BwdParams p) {
  constexpr int NW = 4;
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;        // keys per workgroup
  constexpr int KST = D / 16;
  constexpr int NDB = D / 32;
  constexpr int LDP = D + 8;         // bf16 pitch of K_hat / Q_hat / dO rows
  constexpr int CPR = D / 8;
  constexpr int NQC = BQ / 32;       // 32-row query chunks per block
  constexpr int DSP = BQ + 8;        // bf16 pitch of dS rows (one row per key)
  constexpr int NBLK = NQC * NDB;    // 32x32 blocks of the dQ tile
  constexpr int BPW = NBLK / NW;     // dQ blocks per wave
  static_assert(NBLK % NW == 0, "dQ tile must split evenly over the waves");
  static_assert((BK * CPR) % NT == 0 && (BQ * CPR) % NT == 0, "tiles must split evenly");

  __shared__ __attribute__((aligned(16))) bf16 Ks[BK * LDP];
  __shared__ __attribute__((aligned(16))) bf16 Qs[BQ * LDP];
  __shared__ __attribute__((aligned(16))) bf16 dOs[BQ * LDP];
  __shared__ __attribute__((aligned(16))) bf16 dSs[BK * DSP];
  __shared__ __attribute__((aligned(16))) float lse2s[BQ];
  __shared__ __attribute__((aligned(16))) float dls[BQ];
  __shared__ float rks[BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int T = p.T;
  const int W = p.window;
  const long qstride = (long)p.Hq * D;
  const long kvstride = (long)p.Hkv * D;

  // key blocks in ascending order: the first blocks see the most queries
  const int bid = blockIdx.x;
  const int kb = bid / (p.B * p.Hkv);
  const int g = (bid / p.B) % p.Hkv;
  const int b = bid % p.B;
  const int kb0 = kb * BK;
  const int kw0 = kb0 + 32 * wave;  // first key of this wave
  const int key = kw0 + l32;

  // ---- K_hat block into LDS (RMS-normed), rstd per key
  {
    const bf16* kbase = (const bf16*)p.k + (long)b * T * kvstride + (long)g * D;
#pragma unroll
    for (int i = 0; i < BK * CPR / NT; ++i) {
      const int c = tid + NT * i;
      const int kt = c / CPR;
      const int off = 8 * (c % CPR);
      u32x4 w = {0u, 0u, 0u, 0u};
      if (kb0 + kt < T) w = ld16(kbase + (long)(kb0 + kt) * kvstride + off);
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
      *(u32x4*)&Ks[kt * LDP + off] = w;
    }
  }
  // ---- V fragment (B operand of dP = dO V^T): key l32 of this wave, head_dim 16kk + 8half + 0..7
  bf16x8 vf[KST];
  {
    const bf16* src = (const bf16*)p.v + ((long)b * T + key) * kvstride + (long)g * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (key < T) w = ld16(src + 16 * kk);
      vf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __syncthreads();
  bf16x8 kf[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) kf[kk] = *(const bf16x8*)&Ks[(32 * wave + l32) * LDP + 16 * kk + 8 * half];

  f32x16 dv_acc[NDB], dk_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv_acc[db][r] = 0.f;
      dk_acc[db][r] = 0.f;
    }

  // query blocks whose rows can see at least one key of this block
  const int q_lo = kb0;
  const int q_hi = (W < 0) ? T - 1 : min(T - 1, kb0 + BK - 1 + W);
  const int qb_lo = q_lo / BQ;
  const int qb_hi = q_hi / BQ;

  // transposed-read lane addressing (see sa_common.h)
  const int tr_row = 8 * half + ((lane >> 2) & 3);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int hh = 0; hh < p.G; ++hh) {
    const int head = g * p.G + hh;
    const bf16* qbase = (const bf16*)p.q + (long)b * T * qstride + (long)head * D;
    const bf16* dobase = (const bf16*)p.dout + (long)b * T * qstride + (long)head * D;
    const float* lse_row = p.lse + ((long)b * p.Hq + head) * T;
    const float* dl_row = p.delta + ((long)b * p.Hq + head) * T;
    for (int qb = qb_lo; qb <= qb_hi; ++qb) {
      const int qbase_row = qb * BQ;
      __syncthreads();  // previous block's readers of Qs / dOs / dSs are done
#pragma unroll
      for (int i = 0; i < BQ * CPR / NT; ++i) {
        const int c = tid + NT * i;
        const int qt = c / CPR;
        const int off = 8 * (c % CPR);
        const int qrow = qbase_row + qt;
        u32x4 wq = {0u, 0u, 0u, 0u}, wd = {0u, 0u, 0u, 0u};
        if (qrow < T) {
          wq = ld16(qbase + (long)qrow * qstride + off);
          wd = ld16(dobase + (long)qrow * qstride + off);
        }
        if constexpr (NORM) {
          float x[8];
          unpack8(wq, x);
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
          const float r = fast_rsqrt(group_sum<CPR>(ss) * (1.f / D) + p.eps);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= r;
          wq = pack8(x);
        }
        *(u32x4*)&Qs[qt * LDP + off] = wq;
        *(u32x4*)&dOs[qt * LDP + off] = wd;
      }
      if (tid < BQ) {
        const int qrow = qbase_row + tid;
        lse2s[tid] = qrow < T ? lse_row[qrow] * kLog2e : INFINITY;
        dls[tid] = qrow < T ? dl_row[qrow] : 0.f;
      }
      __syncthreads();

#pragma unroll
      for (int qc = 0; qc < NQC; ++qc) {
        const int q0 = qbase_row + 32 * qc;
        const bool act = !(q0 + 31 < kw0 || (W >= 0 && q0 > kw0 + 31 + W));
        if (!act) continue;
        const bool edge = !(q0 >= kw0 + 31 && (W < 0 || q0 + 31 - kw0 <= W)) || q0 + 31 >= T;
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const bf16* qp = Qs + (32 * qc + swap23(l32)) * LDP + 8 * half;
        const bf16* dop = dOs + (32 * qc + swap23(l32)) * LDP + 8 * half;
#pragma unroll
        for (int kk = 0; kk < KST; ++kk) {
          s = mfma32(*(const bf16x8*)(qp + 16 * kk), kf[kk], s);
          dp = mfma32(*(const bf16x8*)(dop + 16 * kk), vf[kk], dp);
        }
        // register r of this lane: query q0 + 16(r>>3) + 8half + (r&7), key `key`
        float pr[16], ds[16];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int qo = 32 * qc + 16 * ks + 8 * half;
          const f32x4 l0 = *(const f32x4*)&lse2s[qo];
          const f32x4 l1 = *(const f32x4*)&lse2s[qo + 4];
          const f32x4 d0 = *(const f32x4*)&dls[qo];
          const f32x4 d1 = *(const f32x4*)&dls[qo + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 8 * ks + e;
            const float lv = e < 4 ? l0[e] : l1[e - 4];
            const float dv = e < 4 ? d0[e] : d1[e - 4];
            float pe = fast_exp2(s[r] * p.c1 - lv);
            if (edge) {
              const int q = q0 + 16 * ks + 8 * half + e;
              const bool ok = key <= q && q < T && (W < 0 || q - key <= W);
              pe = ok ? pe : 0.f;
            }
            pr[r] = pe;
            ds[r] = pe * (dp[r] - dv);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pack8(pr + 8 * ks));
          const bf16x8 dsb = __builtin_bit_cast(bf16x8, pack8(ds + 8 * ks));
          const int rbase = (32 * qc + 16 * ks + tr_row) * LDP + tr_col;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 a_do = cat(lds_read_tr(dOs + rbase + 32 * db), lds_read_tr(dOs + rbase + 32 * db + 4 * LDP));
            dv_acc[db] = mfma32(a_do, pb, dv_acc[db]);
            const bf16x8 a_q = cat(lds_read_tr(Qs + rbase + 32 * db), lds_read_tr(Qs + rbase + 32 * db + 4 * LDP));
            dk_acc[db] = mfma32(a_q, dsb, dk_acc[db]);
          }
          // dS rows of this lane's key: 8 consecutive queries 32qc + 16ks + 8half + 0..7
          *(u32x4*)&dSs[(32 * wave + l32) * DSP + 32 * qc + 16 * ks + 8 * half] = pack8(ds + 8 * ks);
        }
      }
      __syncthreads();

      // ---- dQ_hat[q][d] += scale * sum_key dS[q][key] K_hat[key][d] over the 128 keys
#pragma unroll
      for (int bi = 0; bi < BPW; ++bi) {
        const int blk = wave * BPW + bi;
        const int qc = blk / NDB;
        const int db = blk % NDB;
        const int q0 = qbase_row + 32 * qc;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        bool any = false;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
          const int kw = kb0 + 32 * (ks / 2);  // first key of the wave that wrote these dS rows
          const bool act = !(q0 + 31 < kw || (W >= 0 && q0 > kw + 31 + W));
          if (!act) continue;
          any = true;
          const bf16* ap = dSs + (16 * ks + tr_row) * DSP + 32 * qc + tr_col;
          const bf16* bp = Ks + (16 * ks + tr_row) * LDP + 32 * db + tr_col;
          const bf16x8 a = cat(lds_read_tr(ap), lds_read_tr(ap + 4 * DSP));
          const bf16x8 bb = cat(lds_read_tr(bp), lds_read_tr(bp + 4 * LDP));
          acc = mfma32(a, bb, acc);
        }
        if (!any) continue;
        // accumulator: column = head_dim 32db + l32, row = query q0 + 8i + 4half + j
        float* dst = p.dq_acc + ((long)b * T + q0 + 4 * half) * qstride + (long)head * D + 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qo = 8 * (r >> 2) + (r & 3);
          if (q0 + 4 * half + qo < T) unsafeAtomicAdd(dst + (long)qo * qstride, p.scale * acc[r]);
        }
      }
    }
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
  hipLaunchKernelGGL((attn_bwd_pre_kernel<D>), dim3(row_blocks), dim3(256), 0, stream, p);
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
