// C ABI of libsa_attn.so (declared in include/sa_attn.h).
//
// Every entry point validates all of its arguments before touching the HIP
// runtime, so an error return means nothing was enqueued, and the
// validation paths run on a host without a GPU.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "sa_attn.h"
#include "sa_kernels.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kAbiVersion = 7;

// Benchmarking hook: events recorded around a kernel of later calls made
// from this host thread (see sa_set_timing_events).
thread_local sa::TimingEvents tl_events[5];
// Testing hook: cap on the workgroups of a persistent launch (0 = none).
thread_local int tl_max_wg = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
bool valid_dim(int d) { return d == 64 || d == 128; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the current device (cached per device). 0 on a runtime error.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Workgroups of a persistent launch: one per compute unit, or the cap set
// with sa_set_max_workgroups. 0 on a runtime error.
int persistent_wgs() {
  const int n = cu_count();
  return (tl_max_wg > 0 && tl_max_wg < n) ? tl_max_wg : n;
}


// Validates the shape arguments shared by the forward and the backward.
sa_status check_shape(int B, int T, int Hq, int Hkv, int head_dim, int window, float scale, float eps) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0) return SA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SA_ERR_SHAPE;
  if (window < -1) return SA_ERR_SHAPE;
  if (!isfinite(scale) || !isfinite(eps) || eps < 0.f) return SA_ERR_SHAPE;
  // element offsets are computed in 64-bit; grids in 32-bit
  const double elems = (double)B * T * (double)Hq * 128.0;
  if (elems > 9.0e18) return SA_ERR_SHAPE;
  if ((double)B * Hq * ((T + 127) / 128) > 2.0e9) return SA_ERR_SHAPE;
  // one batch's rows of q (or k, v) are addressed with 32-bit byte offsets,
  // including the rows of the last 256-row block that lie past T
  if (((double)T + 256.0) * Hq * 128.0 * 2.0 >= 2147483648.0) return SA_ERR_SHAPE;
  if (!valid_dim(head_dim)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

// Logits are bounded by |scale| * D when q and k rows are normed (each normed
// row has Euclidean norm below sqrt(D)); 2% margin covers bf16 rounding of
// the normed rows. A fixed maximum is safe while exp2 of the widest logit
// gap, 2 * bound * log2(e), stays far inside the fp32 normal range.
bool fixed_max_ok(int qk_norm, float scale, int head_dim, float* c2) {
  const float bound = fabsf(scale) * (float)head_dim * 1.02f;
  *c2 = bound * 1.4426950408889634f;
  return qk_norm != 0 && bound <= 32.f;
}

// Validates optional rotary tables: both or neither pointer, rows of at least
// head_dim/2 floats at a 16-byte-aligned stride, and only with the QK-norm.
sa_status check_rope(const float* cos, const float* sin, int stride, int T, int head_dim, int qk_norm,
                     sa::Rope* out) {
  *out = sa::Rope{nullptr, nullptr, 0};
  if (cos == nullptr && sin == nullptr) return SA_OK;
  if (cos == nullptr || sin == nullptr) return SA_ERR_NULL;
  if (!qk_norm) return SA_ERR_UNSUPPORTED;
  if (stride < head_dim / 2 || stride % 4 != 0) return SA_ERR_SHAPE;
  if ((double)T * stride * 4.0 >= 2147483648.0) return SA_ERR_SHAPE;  // 32-bit table offsets
  if (!aligned16(cos) || !aligned16(sin)) return SA_ERR_ALIGN;
  *out = sa::Rope{cos, sin, stride};
  return SA_OK;
}

// Validates optional value-embedding inputs: all four or none; x rows of
// x_stride >= 32 elements (a multiple of 8), 16-byte aligned x, w and table,
// 4-byte aligned ids; the table addressed with 32-bit offsets; only on the
// QK-norm kernels (the forward's key/value prologue mixes the rows).
sa_status check_ve(const void* x, int64_t x_stride, const void* w, const int32_t* ids, const void* table, int vocab,
                   int Hkv, int head_dim, int qk_norm, sa::VeParams* out, uint32_t* table_bytes) {
  *out = sa::VeParams{nullptr, 0, nullptr, nullptr, nullptr};
  *table_bytes = 0;
  const int given = (x != nullptr) + (w != nullptr) + (ids != nullptr) + (table != nullptr);
  if (given == 0) return SA_OK;
  if (given != 4) return SA_ERR_NULL;
  if (!qk_norm) return SA_ERR_UNSUPPORTED;
  if (vocab <= 0 || x_stride < 32 || x_stride % 8 != 0) return SA_ERR_SHAPE;
  if (Hkv > sa::kVeMaxHeads) return SA_ERR_UNSUPPORTED;
  if ((double)vocab * Hkv * head_dim * 2.0 >= 2147483648.0) return SA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(table) || !aligned4(ids)) return SA_ERR_ALIGN;
  *out = sa::VeParams{x, (long)x_stride, w, ids, table};
  *table_bytes = (uint32_t)((size_t)vocab * Hkv * head_dim * 2);
  return SA_OK;
}

size_t ve_blocks(int B, int T) { return ((size_t)B * T + sa::kVeRows - 1) / sa::kVeRows; }

}  // namespace

// Scratch of the backward's no-allocation entry point: one copy per GPU the
// library runs on, held until the process ends. Host code never uses this
// name as an address (on the host it is only a stand-in for the symbol);
// the per-device address comes from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = (size_t)80 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device with that device current. nullptr on a runtime error.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

SA_API int sa_abi_version(void) { return kAbiVersion; }

SA_API size_t sa_attn_ve_workspace_bytes(int B, int T, int Hkv, int head_dim) {
  if (check_shape(B, T, Hkv, Hkv, head_dim, -1, 1.f, 0.f) != SA_OK) return 0;
  const size_t rh = (size_t)B * T * Hkv;
  // v' (bf16), the gate (fp32 per row and head), per-block partial sums of dw
  return round256(rh * head_dim * 2) + round256(rh * 4) + round256(ve_blocks(B, T) * Hkv * 32 * 4);
}

SA_API const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: invalid size, head ratio, window or scalar argument";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: head_dim must be 64 or 128";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE: workspace missing or too small";
    case SA_ERR_HIP: return "SA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown sa_status";
  }
}

SA_API sa_status sa_qknorm(const void* x, void* y, float* rstd, int64_t rows, int head_dim, float eps,
                           void* stream) {
  if (rows < 0 || !isfinite(eps) || eps < 0.f) return SA_ERR_SHAPE;
  if (!valid_dim(head_dim)) return SA_ERR_UNSUPPORTED;
  if (rows == 0) return SA_OK;
  if (x == nullptr || y == nullptr) return SA_ERR_NULL;
  if (!aligned16(x) || !aligned16(y) || (rstd != nullptr && !aligned4(rstd))) return SA_ERR_ALIGN;
  if (rows > (int64_t)1 << 56) return SA_ERR_SHAPE;
  sa::NormParams p{x, y, rstd, rows, eps};
  return sa::launch_qknorm(p, head_dim, (hipStream_t)stream, sa::TimingEvents{}) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// The forward's workspace, which the backward may read back: bf16 normed k
// rows [B,T,Hkv,D], fp32 1/rms of the k rows [B,T,Hkv], and with value
// embeddings the mixed value rows v' [B,T,Hkv,D] (bf16) and the gate [B,T,Hkv].
struct FwdWorkspace {
  char* khat;
  float* rstd_k;
  char* v_mixed;
  float* gate;
};
FwdWorkspace fwd_workspace_of(const void* base, int B, int T, int Hkv, int head_dim) {
  const size_t rh = (size_t)B * T * Hkv;
  FwdWorkspace w;
  w.khat = (char*)base;
  w.rstd_k = (float*)(w.khat + round256(rh * head_dim * 2));
  w.v_mixed = (char*)w.rstd_k + round256(rh * 4);
  w.gate = (float*)(w.v_mixed + round256(rh * head_dim * 2));
  return w;
}

SA_API size_t sa_attn_fwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim) {
  if (check_shape(B, T, Hq, Hkv, head_dim, -1, 1.f, 0.f) != SA_OK) return 0;
  const size_t rh = (size_t)B * T * Hkv;
  return 2 * round256(rh * head_dim * 2) + 2 * round256(rh * 4);
}

static sa_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                          size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                          float softmax_scale, int qk_norm, float eps, const float* rope_cos, const float* rope_sin,
                          int rope_stride, const void* ve_x, int64_t ve_x_stride, const void* ve_w,
                          const int32_t* ve_ids, const void* ve_table, int ve_vocab, void* stream) {
  const sa_status st = check_shape(B, T, Hq, Hkv, head_dim, window, softmax_scale, eps);
  if (st != SA_OK) return st;
  sa::Rope rope;
  const sa_status sr = check_rope(rope_cos, rope_sin, rope_stride, T, head_dim, qk_norm, &rope);
  if (sr != SA_OK) return sr;
  sa::VeParams ve;
  uint32_t ve_bytes = 0;
  const sa_status sv = check_ve(ve_x, ve_x_stride, ve_w, ve_ids, ve_table, ve_vocab, Hkv, head_dim, qk_norm, &ve, &ve_bytes);
  if (sv != SA_OK) return sv;
  if (!q || !k || !v || !o || !lse) return SA_ERR_NULL;
  if (qk_norm && (workspace == nullptr || workspace_bytes < sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, head_dim) ||
                  ((uintptr_t)workspace & 255u) != 0))
    return SA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse)) return SA_ERR_ALIGN;

  sa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.window = (window >= T - 1) ? -1 : window;
  p.c1 = softmax_scale * 1.4426950408889634f;
  p.eps = eps;
  const bool fixed = fixed_max_ok(qk_norm, softmax_scale, head_dim, &p.c2);
  p.khat = k;
  const hipStream_t s = (hipStream_t)stream;
  if (fixed) {
    // two warp groups per workgroup: two query heads of a KV group, or (odd G)
    // two interleaved halves of 256 rows of one head
    p.pair_rows = p.G % 2 != 0;
    p.nsub = p.pair_rows ? p.G : p.G / 2;
    p.nqb = p.pair_rows ? (T + 255) / 256 : (T + 127) / 128;
    p.nwg = persistent_wgs();
    if (p.nwg <= 0) return SA_ERR_HIP;
    // norm pass: normed (and turned) k rows and their 1/rms, which the attention kernel
    // copies as tiles and the backward can reuse; with value embeddings the mixed rows v'
    // and the gate, on which the attention (and the backward) runs
    const FwdWorkspace fw = fwd_workspace_of(workspace, B, T, Hkv, head_dim);
    sa::NormParams np{k, fw.khat, fw.rstd_k, (int64_t)B * T * Hkv, eps, rope, Hkv, T};
    const sa::VePrepParams vp{ve, v, fw.v_mixed, fw.gate, (long)B * T, Hkv, ve_bytes};
    if (sa::launch_qknorm(np, head_dim, s, tl_events[SA_KERNEL_FWD_KNORM], ve.x != nullptr ? &vp : nullptr) !=
        hipSuccess)
      return SA_ERR_HIP;
    p.khat = fw.khat;
    p.vrows = ve.x != nullptr ? fw.v_mixed : v;
    p.rope = rope;
    return sa::launch_fwd_pp(p, head_dim, s, tl_events[SA_KERNEL_FWD]) == hipSuccess ? SA_OK : SA_ERR_HIP;
  }
  // online-softmax kernel (logits without the QK-norm bound); no rotary tables or value embeddings there
  if (rope.cos != nullptr || ve.x != nullptr) return SA_ERR_UNSUPPORTED;
  const int hpw = (p.G % 2 == 0) ? 2 : 1;
  p.nsub = p.G / hpw;
  p.nqb = (T + 127) / 128;
  return sa::launch_fwd(p, head_dim, hpw, qk_norm != 0, fixed, s, tl_events[SA_KERNEL_FWD]) == hipSuccess
             ? SA_OK
             : SA_ERR_HIP;
}

SA_API size_t sa_attn_bwd_workspace_bytes(int B, int T, int Hq, int Hkv, int head_dim) {
  if (check_shape(B, T, Hq, Hkv, head_dim, -1, 1.f, 0.f) != SA_OK) return 0;
  const size_t rows = (size_t)B * T * Hq;
  // bf16 normed q rows, fp32 Delta, fp32 base-2 LSE, bf16 normed k rows, fp32 1/rms of the k rows
  return round256(rows * head_dim * 2) + 2 * round256(rows * sizeof(float)) +
         round256((size_t)B * T * Hkv * head_dim * 2) + round256((size_t)B * T * Hkv * sizeof(float));
}

static sa_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          const void* fwd_workspace, size_t fwd_workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window, float softmax_scale, int qk_norm,
                          float eps, const float* rope_cos, const float* rope_sin, int rope_stride, const void* ve_x,
                          int64_t ve_x_stride, const void* ve_w, const int32_t* ve_ids, const void* ve_table,
                          int ve_vocab, void* dve, float* dve_w, float* dve_x32, void* ve_workspace,
                          size_t ve_workspace_bytes, void* stream) {
  const sa_status st = check_shape(B, T, Hq, Hkv, head_dim, window, softmax_scale, eps);
  if (st != SA_OK) return st;
  sa::Rope rope;
  const sa_status sr = check_rope(rope_cos, rope_sin, rope_stride, T, head_dim, qk_norm, &rope);
  if (sr != SA_OK) return sr;
  sa::VeParams ve;
  uint32_t ve_bytes = 0;
  const sa_status sv = check_ve(ve_x, ve_x_stride, ve_w, ve_ids, ve_table, ve_vocab, Hkv, head_dim, qk_norm, &ve, &ve_bytes);
  if (sv != SA_OK) return sv;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return SA_ERR_NULL;
  if (ve.x != nullptr) {
    if (!dve || !dve_w || !dve_x32) return SA_ERR_NULL;
    if (!aligned16(dve) || !aligned4(dve_w) || !aligned4(dve_x32)) return SA_ERR_ALIGN;
    if (ve_workspace == nullptr || ve_workspace_bytes < sa_attn_ve_workspace_bytes(B, T, Hkv, head_dim) ||
        ((uintptr_t)ve_workspace & 255u) != 0)
      return SA_ERR_WORKSPACE;
  }
  const size_t need = sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, head_dim);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SA_ERR_WORKSPACE;
  if (fwd_workspace != nullptr) {
    // only the QK-norm forward with the fixed row maximum writes what the backward reads back
    float c2 = 0.f;
    if (!fixed_max_ok(qk_norm, softmax_scale, head_dim, &c2)) return SA_ERR_UNSUPPORTED;
    if (fwd_workspace_bytes < sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, head_dim) ||
        ((uintptr_t)fwd_workspace & 255u) != 0)
      return SA_ERR_WORKSPACE;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SA_ERR_ALIGN;

  sa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const size_t rows = (size_t)B * T * Hq;
  p.qhat = qk_norm ? workspace : (void*)q;
  p.delta = (float*)((char*)workspace + round256(rows * head_dim * 2));
  p.lse2 = (float*)((char*)p.delta + round256(rows * sizeof(float)));
  p.B = B;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.window = (window >= T - 1) ? -1 : window;
  p.scale = softmax_scale;
  p.c1 = softmax_scale * 1.4426950408889634f;
  p.eps = eps;
  // dQ: two warp groups per workgroup, on two query heads of a KV group or
  // (odd G) on two interleaved halves of 256 rows of one head
  p.pair_rows = p.G % 2 != 0;
  p.nsub = p.pair_rows ? p.G : p.G / 2;
  p.nqb = p.pair_rows ? (T + 255) / 256 : (T + 127) / 128;
  p.nkb = (T + 127) / 128;
  p.nwg = persistent_wgs();
  if (p.nwg <= 0) return SA_ERR_HIP;
  const hipStream_t s = (hipStream_t)stream;
  p.khat = k;
  const FwdWorkspace fw = fwd_workspace_of(fwd_workspace, B, T, Hkv, head_dim);
  // value embeddings: the attention kernels run on v' = v + g ve, written once (by the
  // forward's norm pass, or below with the k rows)
  const long nrows = (long)B * T;
  const size_t rh = (size_t)nrows * Hkv;
  char* vw = (char*)ve_workspace;
  void* v_mixed = fwd_workspace != nullptr ? fw.v_mixed : vw;
  float* gate = fwd_workspace != nullptr ? fw.gate : (float*)(vw + round256(rh * head_dim * 2));
  float* part = (float*)(vw + round256(rh * head_dim * 2) + round256(rh * 4));
  if (ve.x != nullptr) p.v = v_mixed;
  if (fwd_workspace != nullptr) {
    // the forward's normed k rows and their 1/rms
    p.khat = fw.khat;
    p.rstd_k = fw.rstd_k;
  } else if (qk_norm) {
    // normed k rows, copied straight into LDS as tiles by the dQ kernel (and v', g)
    void* khat = (char*)workspace + round256(rows * head_dim * 2) + 2 * round256(rows * sizeof(float));
    float* rstd_k = (float*)((char*)khat + round256((size_t)B * T * Hkv * head_dim * 2));
    sa::NormParams np{k, khat, rstd_k, (int64_t)B * T * Hkv, eps, rope, Hkv, T};
    const sa::VePrepParams vp{ve, v, v_mixed, gate, nrows, Hkv, ve_bytes};
    if (sa::launch_qknorm(np, head_dim, s, tl_events[SA_KERNEL_BWD_KNORM], ve.x != nullptr ? &vp : nullptr) !=
        hipSuccess)
      return SA_ERR_HIP;
    p.khat = khat;
    p.rstd_k = rstd_k;
  }
  p.rope = rope;
  if (sa::launch_bwd_dq_pp(p, head_dim, s, tl_events[SA_KERNEL_BWD_DQ]) != hipSuccess) return SA_ERR_HIP;
  if (sa::launch_bwd_dkdv_pp(p, head_dim, s, tl_events[SA_KERNEL_BWD_DKDV]) != hipSuccess) return SA_ERR_HIP;
  if (ve.x != nullptr) {
    // dv holds dL/dv' (also the raw v's gradient); the gate's and embedding's gradients from it
    sa::VeBwdParams bp{ve, dv, gate, dve, dve_x32, part, dve_w, nrows, Hkv, ve_bytes};
    if (sa::launch_ve_bwd(bp, head_dim, s) != hipSuccess) return SA_ERR_HIP;
  }
  return SA_OK;
}

SA_API sa_status sa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                             float softmax_scale, int qk_norm, float eps, void* stream) {
  return attn_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, T, Hq, Hkv, head_dim, window, softmax_scale,
                  qk_norm, eps, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, 0, stream);
}

SA_API sa_status sa_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                                  size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                                  float softmax_scale, int qk_norm, float eps, const float* rope_cos,
                                  const float* rope_sin, int rope_stride, void* stream) {
  if (rope_cos == nullptr || rope_sin == nullptr) return SA_ERR_NULL;
  return attn_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, T, Hq, Hkv, head_dim, window, softmax_scale,
                  qk_norm, eps, rope_cos, rope_sin, rope_stride, nullptr, 0, nullptr, nullptr, nullptr, 0, stream);
}

SA_API sa_status sa_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                                size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                                float softmax_scale, int qk_norm, float eps, const float* rope_cos,
                                const float* rope_sin, int rope_stride, const void* ve_x, int64_t ve_x_stride,
                                const void* ve_w, const int32_t* ve_ids, const void* ve_table, int ve_vocab,
                                void* stream) {
  return attn_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, T, Hq, Hkv, head_dim, window, softmax_scale,
                  qk_norm, eps, rope_cos, rope_sin, rope_stride, ve_x, ve_x_stride, ve_w, ve_ids, ve_table, ve_vocab,
                  stream);
}

SA_API sa_status sa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                             float softmax_scale, int qk_norm, float eps, void* stream) {
  return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, nullptr, 0, B, T, Hq, Hkv, head_dim, window,
                  softmax_scale, qk_norm, eps, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr,
                  nullptr, nullptr, nullptr, 0, stream);
}

SA_API size_t sa_attn_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

SA_API sa_status sa_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                     const void* dout, void* dq, void* dk, void* dv, int B, int T, int Hq, int Hkv,
                                     int head_dim, int window, float softmax_scale, int qk_norm, float eps,
                                     void* stream) {
  // everything that can be checked without the runtime first
  const sa_status st = check_shape(B, T, Hq, Hkv, head_dim, window, softmax_scale, eps);
  if (st != SA_OK) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return SA_ERR_ALIGN;
  if (sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, head_dim) > kScratchBytes) return SA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (ws == nullptr) return SA_ERR_HIP;
  return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, nullptr, 0, B, T, Hq, Hkv, head_dim, window,
                  softmax_scale, qk_norm, eps, nullptr, nullptr, 0, nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr,
                  nullptr, nullptr, nullptr, 0, stream);
}

SA_API sa_status sa_attn_bwd_rope(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                  size_t workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                                  float softmax_scale, int qk_norm, float eps, const float* rope_cos,
                                  const float* rope_sin, int rope_stride, void* stream) {
  if (rope_cos == nullptr || rope_sin == nullptr) return SA_ERR_NULL;
  return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, nullptr, 0, B, T, Hq, Hkv, head_dim, window,
                  softmax_scale, qk_norm, eps, rope_cos, rope_sin, rope_stride, nullptr, 0, nullptr, nullptr, nullptr,
                  0, nullptr, nullptr, nullptr, nullptr, 0, stream);
}

SA_API sa_status sa_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                size_t workspace_bytes, const void* fwd_workspace, size_t fwd_workspace_bytes, int B, int T, int Hq, int Hkv, int head_dim, int window,
                                float softmax_scale, int qk_norm, float eps, const float* rope_cos,
                                const float* rope_sin, int rope_stride, const void* ve_x, int64_t ve_x_stride,
                                const void* ve_w, const int32_t* ve_ids, const void* ve_table, int ve_vocab,
                                void* dve, float* dve_w, float* dve_x32, void* ve_workspace,
                                size_t ve_workspace_bytes, void* stream) {
  return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, fwd_workspace, fwd_workspace_bytes,
                  B, T, Hq, Hkv, head_dim, window,
                  softmax_scale, qk_norm, eps, rope_cos, rope_sin, rope_stride, ve_x, ve_x_stride, ve_w, ve_ids,
                  ve_table, ve_vocab, dve, dve_w, dve_x32, ve_workspace, ve_workspace_bytes, stream);
}

// ---------------------------------------------------------------- polar express

namespace {

// [guide] 8.2.3, the printed coefficients (a, b, c) of the five steps, in order.
constexpr float kPolarCoeffs[5][3] = {
    {8.156554524902461f, -22.48329292557795f, 15.878769915207462f},
    {4.042929935166739f, -2.808917465908714f, 0.5000178451051316f},
    {3.8916678022926607f, -2.772484153217685f, 0.5060648178503393f},
    {3.285753657755655f, -2.3681294933425376f, 0.46449024233003106f},
    {2.3465413258596377f, -1.7097828382687081f, 0.42323551169305323f},
};

sa_status check_polar(int batch, int rows, int cols, int steps, float eps) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return SA_ERR_SHAPE;
  if (rows % 128 != 0 || cols % 128 != 0) return SA_ERR_UNSUPPORTED;
  if ((double)rows * cols * 2.0 >= 2147483648.0 || (double)batch * rows * cols > 9.0e18) return SA_ERR_SHAPE;
  if (batch > 65535) return SA_ERR_SHAPE;
  // one-dimensional GEMM grids: batch x tiles x (at most 8 K splits) x 256 threads below 2^31
  if ((long)batch * (rows / 128) * (cols / 128) >= (1L << 20)) return SA_ERR_SHAPE;
  if (steps < 1 || steps > 5) return SA_ERR_SHAPE;
  if (!isfinite(eps) || eps < 0.f) return SA_ERR_SHAPE;
  return SA_OK;
}

// K splits of a GEMM with `jobs` workgroups (computed tiles x batch): the
// fewest equal ranges (multiples of 64, at least 1024 long) that give 512
// workgroups, enough to fill the compute units twice over. Shorter ranges
// do not pay for the partial tiles' round trip through memory (measured on
// the trainer's groups: K = 3072 in 3 ranges beat 2 and 4; K = 768 unsplit
// beat 3 ranges).
int polar_splits(long jobs, int K) {
  int best = 1;
  for (int sp : {1, 2, 3, 4, 6, 8}) {
    if (K % (64 * sp) != 0 || K / sp < 1024) continue;
    best = sp;
    if (jobs * sp >= 512) break;
  }
  return best;
}

// Tile of an unsplit polar-express product C [M][N] (K a multiple of 128): the shape whose
// rounds of workgroups (two per compute unit) take the least time, a round's time taken as
// the tile's area over its relative rate per element, measured at m = 768 (K = 768): on B X,
// 128 x 128 1 (19.3 us per round), 96 x 128 0.81 (B given as [K][N] only; 17.9 us), 192 x 192
// 0.85 (50.9 us); on A A of 8 matrices, 64 x 64 0.26 (one round of 624 tiles, 14.1 us, against
// 14.8 for one of 168 tiles of 128 x 128).
int polar_tile(int batch, int M, int N, bool b_kn, bool sym) {
  if (cu_count() <= 0) return 128;  // no device to size the rounds for
  int best = 128;
  double best_cost = 0.0;
  for (int t : {128, 96, 192, 64}) {
    const int tm = t, tn = (t == 192 || t == 64) ? t : 128;
    if (M % tm != 0 || N % tn != 0 || (t == 96 && (!b_kn || sym)) || (t == 64 && b_kn)) continue;
    // workgroups per compute unit: two, or four of the 64 x 64 tile
    const long slots = (t == 64 ? 4L : 2L) * cu_count();
    const long tiles = (long)batch * sa::gemm_tiles(M, N, sym, tm, tn);
    const double rate = t == 128 ? 1.0 : (t == 96 ? 0.81 : (t == 192 ? 0.85 : 0.26));
    const double cost = (double)((tiles + slots - 1) / slots) * tm * tn / rate;
    if (t == 128 || cost < best_cost) {
      best = t;
      best_cost = cost;
    }
  }
  return best;
}

// The two symmetric products of a step on [m][n] matrices: A = X X^T (K = n)
// and A A (K = m), both with upper tiles only; their splits and the floats
// of split partials they need.
struct PolarPlan {
  int s_xx, s_aa;
  size_t part_floats;
};
PolarPlan polar_plan(int batch, int m, int n) {
  const long jobs = (long)sa::gemm_tiles(m, m, 1) * batch;
  PolarPlan pl{polar_splits(jobs, n), polar_splits(jobs, m), 0};
  const int smax = pl.s_xx > pl.s_aa ? pl.s_xx : pl.s_aa;
  pl.part_floats = smax > 1 ? (size_t)jobs * smax * 128 * 128 : 0;
  return pl;
}

// Tiles of one step's three products on [m][n] matrices (tall: the iterate is [n][m]): the Gram
// (128 on the first step, whose epilogue sums the diagonal, when split, and for a tall matrix,
// whose Gram reads both operands as [K][*]), A A, and the X update.
struct PolarTiles {
  int gram, aa, upd;
};
PolarTiles polar_tiles(int batch, int m, int n, bool tall, bool first, const PolarPlan& pl) {
  PolarTiles t;
  t.gram = (pl.s_xx > 1 || first || tall) ? 128 : polar_tile(batch, m, m, false, true);
  t.aa = pl.s_aa > 1 ? 128 : polar_tile(batch, m, m, false, true);
  t.upd = tall ? polar_tile(batch, n, m, false, false) : polar_tile(batch, m, n, true, false);
  return t;
}

}  // namespace

SA_API double sa_polar_express_executed_flops(int batch, int rows, int cols, int steps) {
  if (check_polar(batch, rows, cols, steps, 0.f) != SA_OK) return 0.0;
  const bool tall = rows > cols;
  const int m = tall ? cols : rows, n = tall ? rows : cols;
  const PolarPlan pl = polar_plan(batch, m, n);
  double f = 0.0;
  for (int k = 0; k < steps; ++k) {
    const PolarTiles t = polar_tiles(batch, m, n, tall, k == 0, pl);
    // the symmetric products compute their tiles on and above the diagonal only
    f += (double)sa::gemm_tiles(m, m, 1, t.gram, t.gram) * t.gram * t.gram * 2.0 * n;
    f += (double)sa::gemm_tiles(m, m, 1, t.aa, t.aa) * t.aa * t.aa * 2.0 * m;
    f += 2.0 * m * (double)m * n;
  }
  return f * batch;
}

SA_API size_t sa_polar_express_workspace_bytes(int batch, int rows, int cols) {
  if (check_polar(batch, rows, cols, 5, 0.f) != SA_OK) return 0;
  const size_t m = (size_t)(rows < cols ? rows : cols), n = (size_t)(rows < cols ? cols : rows);
  const PolarPlan pl = polar_plan(batch, (int)m, (int)n);
  // X (two buffers, wide side [m][n]), A and B ([m][m]), partial sums of the
  // first Gram product's diagonal (||G||_F^2), split-K partial tiles
  return 2 * round256((size_t)batch * m * n * 2) + 2 * round256((size_t)batch * m * m * 2) +
         round256((size_t)batch * sa::gemm_trace_parts((int)m) * 4) + round256(pl.part_floats * 4);
}

SA_API sa_status sa_polar_express(const void* g, void* out, void* workspace, size_t workspace_bytes, int batch,
                                  int rows, int cols, int steps, float eps, void* stream) {
  const sa_status st = check_polar(batch, rows, cols, steps, eps);
  if (st != SA_OK) return st;
  if (!g || !out) return SA_ERR_NULL;
  if (!aligned16(g) || !aligned16(out)) return SA_ERR_ALIGN;
  const size_t need = sa_polar_express_workspace_bytes(batch, rows, cols);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return SA_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const bool tall = rows > cols;
  const int m = tall ? cols : rows, n = tall ? rows : cols;
  char* ws = (char*)workspace;
  void* x0 = ws;
  void* x1 = ws + round256((size_t)batch * m * n * 2);
  void* A = (char*)x1 + round256((size_t)batch * m * n * 2);
  void* Bm = (char*)A + round256((size_t)batch * m * m * 2);
  float* part = (float*)((char*)Bm + round256((size_t)batch * m * m * 2));
  const PolarPlan pl = polar_plan(batch, m, n);
  float* kpart = (float*)((char*)part + round256((size_t)batch * sa::gemm_trace_parts(m) * 4));
  // A tall matrix G ([n][m], n > m) is iterated as it is: with Y = G (the transpose of the wide
  // iterate X), A = X X^T = Y^T Y (both operands given as [K][*]) and X <- B X + a X becomes
  // Y <- Y B + a Y (B symmetric, so given as [N][K] it is B itself).
  // step k writes bufs[k % 2]
  void* bufs[2] = {x1, x0};
  const void* cur = g;
  const int parts = sa::gemm_trace_parts(m);
  for (int k = 0; k < steps; ++k) {
    const float a = kPolarCoeffs[k][0], b = kPolarCoeffs[k][1], c = kPolarCoeffs[k][2];
    // On the first step X = s G, s = 1 / (||G||_F + eps): its Gram product is G G^T itself (A0),
    // written with the partial sums of its diagonal (||G||_F^2) in 128 x 128 tiles, and the next
    // two products take the powers of s: B = c s^4 A0 A0 + b s^2 A0, X <- s B G + a s G.
    const bool first = k == 0;
    const float* nsum = first ? part : nullptr;
    // A = X X^T (symmetric: upper tiles only)
    sa::GemmParams pg{cur, cur, nullptr, A, m, m, n, 1.f, 0.f, 1, pl.s_xx, kpart, nullptr, 0, 0, 0, eps,
                      first ? part : nullptr};
    const PolarTiles tl = polar_tiles(batch, m, n, tall, first, pl);
    const int tg = tl.gram;
    if (sa::launch_gemm(pg, tall, batch, s, tg, tall) != hipSuccess) return SA_ERR_HIP;
    // B = c A A + b A  (A is symmetric: A A = A A^T, and so is B)
    sa::GemmParams pb{A, A, A, Bm, m, m, m, c, b, 1, pl.s_aa, kpart, nsum, parts, 4, 2, eps, nullptr};
    if (sa::launch_gemm(pb, false, batch, s, tl.aa) != hipSuccess)
      return SA_ERR_HIP;
    // X <- B X + a X (tall: Y <- Y B + a Y), straight into the output on the last step
    void* dst = k == steps - 1 ? out : bufs[k % 2];
    if (tall) {
      sa::GemmParams py{cur, Bm, cur, dst, n, m, m, 1.f, a, 0, 0, nullptr, nsum, parts, 1, 1, eps, nullptr};
      if (sa::launch_gemm(py, false, batch, s, tl.upd) != hipSuccess)
        return SA_ERR_HIP;
    } else {
      sa::GemmParams px{Bm, cur, cur, dst, m, n, m, 1.f, a, 0, 0, nullptr, nsum, parts, 1, 1, eps, nullptr};
      if (sa::launch_gemm(px, true, batch, s, tl.upd) != hipSuccess) return SA_ERR_HIP;
    }
    cur = bufs[k % 2];
  }
  return SA_OK;
}

SA_API sa_status sa_set_timing_events(int kernel, void* start, void* stop) {
  if (kernel < SA_KERNEL_FWD || kernel > SA_KERNEL_BWD_KNORM) return SA_ERR_SHAPE;
  if ((start == nullptr) != (stop == nullptr)) return SA_ERR_NULL;
  tl_events[kernel].start = (hipEvent_t)start;
  tl_events[kernel].stop = (hipEvent_t)stop;
  return SA_OK;
}

SA_API sa_status sa_set_max_workgroups(int n) {
  if (n < 0) return SA_ERR_SHAPE;
  tl_max_wg = n;
  return SA_OK;
}
