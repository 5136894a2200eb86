// orpo_head.hip — host side of the C ABI declared in include/orpo_head.h: argument validation,
// launch planning (vocabulary splits for the forward, token chunk x vocabulary block for the
// backward) and kernel launches on the caller's stream. No allocation, no host synchronisation
// (except orpo_read_status, which is documented to wait).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/orpo_head.h"
#include "objective_kernels.hpp"

namespace {

using namespace orpo;

thread_local int32_t g_last_hip = 0;

constexpr size_t kHeader = 256;                     // status word + padding at the start of a workspace
constexpr int kMergeWideSplits = 32;                // from this many forward splits, a wave per token merges
constexpr int kTargetWorkgroups = 256;              // forward grid target (one round on 256 CUs)
constexpr int64_t kChunkDefault = 8192;             // backward token chunk C (multiple of 256)
// Default coefficient block: the largest that fits 256 MiB per coefficient buffer, but no wider
// than an eighth of the vocabulary (rounded up to 256) unless that is under 16384 rows, so that a
// small vocabulary still pipelines over several items (the first launch's coefficients and the
// last one's dh/dW share the GPU with nothing).
constexpr int64_t kBvItems = 8, kBvMin = 16384;
constexpr size_t kCoeffDefault = size_t(256) << 20;
int64_t g_chunk = kChunkDefault;
size_t g_coeff_budget = 0;                          // 0: the default block rule above

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

#define ORPO_HIP(x)                                  \
  do {                                               \
    hipError_t e_ = (x);                             \
    if (e_ != hipSuccess) {                          \
      g_last_hip = (int32_t)e_;                      \
      return ORPO_EHIP;                              \
    }                                                \
  } while (0)

inline orpo_status launched() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip = (int32_t)e;
    return ORPO_EHIP;
  }
  return ORPO_OK;
}

// ---- tracing: event pairs around launches ------------------------------------------------
struct TraceRec {
  hipEvent_t start, end;
  int kind;
  double flops;
};
std::vector<TraceRec> g_trace;   // pre-created event pairs
size_t g_trace_used = 0;
bool g_trace_on = false;

// Brackets one launch: `begin` before it, `end` after it (both on the launch's stream).
struct TraceScope {
  TraceRec* rec = nullptr;
  hipStream_t st;
  TraceScope(int kind, double flops, hipStream_t s) : st(s) {
    if (g_trace_on && g_trace_used < g_trace.size()) {
      rec = &g_trace[g_trace_used++];
      rec->kind = kind;
      rec->flops = flops;
      if (hipEventRecord(rec->start, st) != hipSuccess) rec = nullptr;
    }
  }
  ~TraceScope() {
    if (rec) (void)hipEventRecord(rec->end, st);
  }
};

// z = cap (1 - 2 r) is evaluated in fp32 with r = 1 / (1 + e^(2 raw / cap)) near 1/2, so each
// logit carries an absolute error of about cap 2^-22 (2.4e-4 at 1024): beyond that the softcap's
// own rounding would reach the 1e-3 log-prob tolerance. Softcaps up to kFixedRefMaxCap use the
// fixed softmax reference, larger ones the running maximum.
constexpr float kMaxSoftcap = 1024.f;

// Format combinations the library implements.
enum Kind { kF32, kBf16, kQ4, kBad };

orpo_status check_desc(const orpo_head_desc* d, Kind* kind) {
  if (!d) return ORPO_EINVAL;
  if (d->M < 0 || d->d <= 0 || d->V <= 0) return ORPO_EINVAL;
  if (d->V > INT32_MAX || d->M > INT32_MAX || d->d > (int64_t(1) << 20)) return ORPO_EUNSUPPORTED;
  if ((d->flags & ~uint32_t(ORPO_DW_ACCUMULATE | ORPO_DH_BF16)) != 0) return ORPO_EINVAL;
  if (!(d->softcap <= 0.f || d->softcap > 0.f)) return ORPO_EINVAL;   // NaN
  if (d->softcap > kMaxSoftcap) return ORPO_EUNSUPPORTED;
  Kind k = kBad;
  if (d->h_fmt == ORPO_F32 && d->w_fmt == ORPO_F32) k = kF32;
  else if (d->h_fmt == ORPO_BF16 && d->w_fmt == ORPO_BF16) k = kBf16;
  else if (d->h_fmt == ORPO_BF16 && d->w_fmt == ORPO_Q4G64) k = kQ4;
  else if ((d->h_fmt == ORPO_F32 || d->h_fmt == ORPO_BF16) &&
           (d->w_fmt == ORPO_F32 || d->w_fmt == ORPO_BF16 || d->w_fmt == ORPO_Q4G64))
    return ORPO_EUNSUPPORTED;
  else
    return ORPO_EINVAL;
  if (d->d % 64 != 0) return ORPO_EUNSUPPORTED;
  if (!(d->skip_eps >= 0.f) || d->skip_eps == __builtin_huge_valf()) return ORPO_EINVAL;
  if (d->skip_eps > 0.f && k == kF32) return ORPO_EUNSUPPORTED;   // 32-wide K steps, 64-wide blocks
  *kind = k;
  return ORPO_OK;
}

orpo_status check_weight(Kind k, const orpo_weight& W) {
  if (!W.w) return ORPO_EINVAL;
  if (k == kQ4) return (W.scales && W.biases) ? ORPO_OK : ORPO_EINVAL;
  return (W.scales || W.biases) ? ORPO_EINVAL : ORPO_OK;
}

struct FwdPlan {
  int n_tb, nblk, tps, n_vtiles;
  size_t tmax_off;   // byte offset of the per-tile maxima (0: not recorded)
  size_t ws;
};

FwdPlan plan_fwd(const orpo_head_desc* d) {
  FwdPlan p;
  p.n_tb = (int)cdiv(std::max<int64_t>(d->M, 1), kTile);
  p.n_vtiles = (int)cdiv(d->V, kTile);
  int nblk = (int)std::min<int64_t>(p.n_vtiles, std::max<int64_t>(1, cdiv(kTargetWorkgroups, p.n_tb)));
  p.tps = (int)cdiv(p.n_vtiles, nblk);
  p.nblk = (int)cdiv(p.n_vtiles, p.tps);
  p.ws = kHeader + round_up(size_t(p.nblk) * size_t(std::max<int64_t>(d->M, 0)) * sizeof(float2), 256);
  p.tmax_off = 0;
  if (d->skip_eps > 0.f) {   // per tile and wave, the largest raw logit (the backward's cold-tile test)
    p.tmax_off = p.ws;
    p.ws += round_up(size_t(p.n_tb) * size_t(p.n_vtiles) * 8 * sizeof(float), 256);
  }
  return p;
}

struct BwdPlan {
  int64_t C, BVb;
  size_t dh_acc_bytes;   // fp32 [C, d] chunk accumulator for bf16 dh over several blocks (else 0)
  size_t fl_bytes;   // skip flags per coefficient buffer (0 without the coefficient filter)
  int dh_split;      // K ranges per dh tile in a launch with coefficient tiles (1: none)
  int dh_split_last; // ... in the last launch, which holds only dh / dW tiles
  size_t part_off, part_bytes;   // fp32 [max split][C][d] dh partials (a split > 1)
  size_t ws;
};

BwdPlan plan_bwd(const orpo_head_desc* d, Kind k) {
  BwdPlan p;
  const int64_t esize = k == kF32 ? 4 : 2;
  // The backward's loaders address a token chunk of h, a vocabulary block of W and a coefficient
  // buffer each through one buffer descriptor with 32-bit offsets: every one of them is kept
  // within kSpan bytes (never binding at the shapes of the pages; a 256-row tile always fits).
  const int64_t kSpan = int64_t(1) << 31;
  const int64_t row = d->d * esize;
  const int64_t rows_cap = std::max<int64_t>(kTile, kSpan / row / kTile * kTile);
  p.C = std::min<int64_t>(std::min<int64_t>(cdiv(std::max<int64_t>(d->M, 1), kTile) * kTile, g_chunk),
                          rows_cap);
  const size_t budget = g_coeff_budget ? g_coeff_budget : kCoeffDefault;
  int64_t bv = std::max<int64_t>(kTile, int64_t(budget) / (p.C * esize) / kTile * kTile);
  if (!g_coeff_budget) bv = std::min(bv, std::max(kBvMin, cdiv(cdiv(d->V, kBvItems), kTile) * kTile));
  bv = std::min(bv, rows_cap);
  bv = std::min(bv, std::max<int64_t>(kTile, kSpan / (p.C * esize) / kTile * kTile));
  p.BVb = std::min<int64_t>(cdiv(d->V, kTile) * kTile, bv);
  // With the coefficient filter: per buffer, dh flags [C/256][BVb/64][4 waves] and dW flags
  // [BVb/256][C/64][2 waves], one byte each.
  p.fl_bytes = d->skip_eps > 0.f
                   ? round_up(size_t(p.C / kTile) * size_t(p.BVb / 64) * 4 +
                                  size_t(p.BVb / kTile) * size_t(p.C / 64) * 2, 256)
                   : 0;
  p.dh_acc_bytes = (d->flags & ORPO_DH_BF16) && cdiv(d->V, p.BVb) > 1
                       ? round_up(size_t(p.C) * size_t(d->d) * sizeof(float), 256)
                       : 0;
  // Split-K dh. A dh tile's K is the whole vocabulary block, so with few token tiles (small M) a
  // launch holds a few dh tiles that each run far longer than the launch's average work per CU,
  // and the launch waits for them. When a dh tile's K steps reach 1.5 times that average, its K
  // is split over S = ceil(steps / average) workgroups (at most one round of kTargetWorkgroups dh
  // workgroups, at most 16 splits, at least 4 K steps each), so the partials take at most 256
  // tiles x 256 x 256 fp32 = 64 MiB. The average is taken with an item's dh, dW and coefficient
  // tiles for the mixed launches and without the coefficient tiles for the last launch; it assumes
  // dW tiles are present (the workspace size does not know whether dW is asked for).
  {
    const int64_t kbk = k == kF32 ? 32 : 64;
    const int64_t n_jt = cdiv(d->d, kTile), n_tt = cdiv(p.C, kTile), n_vt = cdiv(p.BVb, kTile);
    const int64_t nk_dh = cdiv(p.BVb, kbk), n_dh = n_tt * n_jt;
    const int64_t gemm = n_dh * nk_dh + n_vt * n_jt * cdiv(p.C, kbk);
    auto split_for = [&](int64_t work) {
      const int64_t per_cu = cdiv(work, kTargetWorkgroups);
      if (2 * nk_dh < 3 * per_cu) return 1;
      const int64_t S = std::min<int64_t>(std::min<int64_t>(cdiv(nk_dh, per_cu), kTargetWorkgroups / n_dh),
                                          std::min<int64_t>(16, nk_dh / 4));
      return S >= 2 ? (int)S : 1;
    };
    p.dh_split = split_for(gemm + n_tt * n_vt * cdiv(d->d, kbk));
    p.dh_split_last = split_for(gemm);
  }
  const int s_max = std::max(p.dh_split, p.dh_split_last);
  p.part_bytes = s_max > 1 ? round_up(size_t(s_max) * size_t(p.C) * size_t(d->d) * 4, 256) : 0;
  p.part_off = kHeader + 2 * size_t(p.C) * size_t(p.BVb) * size_t(esize) + 2 * p.fl_bytes;
  p.ws = p.part_off + p.part_bytes + p.dh_acc_bytes;
  return p;
}

// Under the coefficient filter a dh / dW tile lists its K steps (64 entries or tokens each) in LDS.
bool bwd_plan_supported(const orpo_head_desc* d, const BwdPlan& p) {
  return !(d->skip_eps > 0.f) || (p.BVb / 64 <= kMaxKSteps && p.C / 64 <= kMaxKSteps);
}

template <class E, bool Q4, int MODE>
orpo_status launch_fwd_mode(const FwdArgs& a, int grid, hipStream_t st) {
  TraceScope ts(ORPO_K_FWD, 2.0 * double(a.M) * double(a.V) * double(a.d), st);
  // bf16, 4-bit and fp8 heads (the coefficient filter's formats); not the FP8 head's running-max
  // mode, whose extra live state would spill (check_fp8 refuses that combination).
  constexpr bool kTmax = E::kSize <= 2 && !(E::kSize == 1 && MODE == kSoftcapRunMax);
  if constexpr (kTmax) {
    if (a.tmax) {
      hipLaunchKernelGGL((fwd_kernel<E, Q4, MODE, true>), dim3(grid), dim3(kThreads), 0, st, a);
      return launched();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<E, Q4, MODE, false>), dim3(grid), dim3(kThreads), 0, st, a);
  return launched();
}

// The forward's softmax mode for a softcap: none, the fixed reference, or the running maximum.
template <class E, bool Q4>
orpo_status launch_fwd(const FwdArgs& a, int grid, hipStream_t st) {
  if (!(a.cap > 0.f)) return launch_fwd_mode<E, Q4, kNoSoftcap>(a, grid, st);
  if (a.cap <= kFixedRefMaxCap) return launch_fwd_mode<E, Q4, kSoftcapFixed>(a, grid, st);
  return launch_fwd_mode<E, Q4, kSoftcapRunMax>(a, grid, st);
}

template <class E, bool Q4, bool SC, bool F8 = false>
orpo_status launch_bwd(const BwdArgs& a, int grid, hipStream_t st) {
  const double cf = 2.0 * double(a.cf.C_cur) * double(a.cf.BV_cur) * double(a.d) * (a.cf.n_tiles > 0);
  const double gm = (a.gm.n_tiles > a.gm.n_dh ? 4.0 : 2.0) * double(a.gm.C_cur) * double(a.gm.BV_cur) *
                    double(a.d) * (a.gm.n_tiles > 0);
  const int kind = a.gm.n_tiles == 0 ? ORPO_K_COEFF : (a.cf.n_tiles == 0 ? ORPO_K_DHDW : ORPO_K_BWD);
  TraceScope ts(kind, cf + gm, st);
  if constexpr (E::kSize == 2) {   // the coefficient filter exists for bf16 coefficients only
    if (a.skip_eps > 0.f) {
      hipLaunchKernelGGL((bwd_kernel<E, Q4, SC, true, F8>), dim3(grid), dim3(kThreads), 0, st, a);
      return launched();
    }
  }
  hipLaunchKernelGGL((bwd_kernel<E, Q4, SC, false, F8>), dim3(grid), dim3(kThreads), 0, st, a);
  return launched();
}

// FP8 logit operands: a bf16 head, d a multiple of 128 (one 128-byte stage of K per step), and
// all four arrays given.
orpo_status check_fp8(const orpo_head_desc* d, Kind k, const orpo_fp8_operands* q) {
  if (!q) return ORPO_EINVAL;
  if (k != kBf16 || d->d % 128 != 0) return ORPO_EUNSUPPORTED;
  if (d->softcap > kFixedRefMaxCap && d->skip_eps > 0.f) return ORPO_EUNSUPPORTED;
  if (d->M > 0 && (!q->hq || !q->h_exp || !q->wq || !q->w_exp)) return ORPO_EINVAL;
  return ORPO_OK;
}

Q4Weight q4_of(const orpo_head_desc* d, const orpo_weight& W) {
  Q4Weight q;
  q.wq = (const uint32_t*)W.w;
  q.scales = (const uint16_t*)W.scales;
  q.biases = (const uint16_t*)W.biases;
  q.V = d->V;
  q.d = d->d;
  return q;
}

}  // namespace

extern "C" {

size_t orpo_head_fwd_workspace_bytes(const orpo_head_desc* desc) {
  Kind k;
  if (check_desc(desc, &k) != ORPO_OK) return 0;
  return plan_fwd(desc).ws;
}

size_t orpo_head_bwd_workspace_bytes(const orpo_head_desc* desc) {
  Kind k;
  if (check_desc(desc, &k) != ORPO_OK) return 0;
  if ((desc->flags & ORPO_DH_BF16) && k == kF32) return 0;   // unsupported
  const BwdPlan p = plan_bwd(desc, k);
  return bwd_plan_supported(desc, p) ? p.ws : 0;
}

size_t orpo_loss_workspace_bytes(int64_t M, int32_t n_pairs) {
  if (M < 0 || n_pairs < 1) return 0;
  // Up to 3 spans per pair: means, sums, dL/dmean, counts (3P each) and 3P per-pair terms.
  return kHeader + round_up(size_t(n_pairs) * 15 * 8, 256);
}

}  // extern "C"

namespace {

// The forward of either head: `q8` null runs the exact head on h and W, else the FP8 logit
// operands (desc and the checks as in the entry points).
orpo_status fwd_impl(const orpo_head_desc* desc, Kind k, const void* h, const orpo_weight& W,
                     const orpo_fp8_operands* q8, const int32_t* labels, float* logp, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  const FwdPlan p = plan_fwd(desc);
  if (!ws || ws_bytes < p.ws || (uintptr_t)ws % 256) return ORPO_ENOWS;
  if (desc->M == 0) return ORPO_OK;
  if ((!q8 && !h) || !labels || !logp || !lse) return ORPO_EINVAL;

  FwdArgs a{};
  a.h = q8 ? (const void*)q8->hq : h;
  a.w = q8 ? (const void*)q8->wq : W.w;
  a.q4 = q4_of(desc, W);
  a.h_exp = q8 ? q8->h_exp : nullptr;
  a.w_exp = q8 ? q8->w_exp : nullptr;
  a.labels = labels;
  a.logp = logp;
  a.part = (float2*)((char*)ws + kHeader);
  a.tmax = p.tmax_off ? (float*)((char*)ws + p.tmax_off) : nullptr;
  a.status = (uint32_t*)ws;
  a.M = desc->M;
  a.d = desc->d;
  a.V = desc->V;
  a.cap = desc->softcap;
  a.ignore_index = desc->ignore_index;
  a.n_tb = p.n_tb;
  a.nblk = p.nblk;
  a.tiles_per_split = p.tps;
  a.n_vtiles = p.n_vtiles;
  const int grid = p.n_tb * p.nblk;
  orpo_status st;
  if (q8) st = launch_fwd<EFp8, false>(a, grid, stream);
  else if (k == kF32) st = launch_fwd<EF32, false>(a, grid, stream);
  else if (k == kBf16) st = launch_fwd<EBf16, false>(a, grid, stream);
  else st = launch_fwd<EBf16, true>(a, grid, stream);
  if (st != ORPO_OK) return st;
  TraceScope ts(ORPO_K_MERGE, 0.0, stream);
  if (p.nblk >= kMergeWideSplits)   // small M: many splits per token, one wave per token
    hipLaunchKernelGGL(merge_wide_kernel, dim3((unsigned)cdiv(desc->M, 4)), dim3(256), 0, stream,
                       (const float2*)a.part, p.nblk, desc->M, labels, desc->V, desc->ignore_index,
                       logp, lse, a.status);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)cdiv(desc->M, 256)), dim3(256), 0, stream,
                       (const float2*)a.part, p.nblk, desc->M, labels, desc->V, desc->ignore_index,
                       logp, lse, a.status);
  return launched();
}

}  // namespace

extern "C" {

orpo_status orpo_head_fwd(const orpo_head_desc* desc, const void* h, orpo_weight W,
                          const int32_t* labels, float* logp, float* lse, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  Kind k;
  orpo_status st = check_desc(desc, &k);
  if (st != ORPO_OK) return st;
  if ((st = check_weight(k, W)) != ORPO_OK) return st;
  return fwd_impl(desc, k, h, W, nullptr, labels, logp, lse, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// The allocation-free forward's workspace: one file-scope array per GPU, held until the process
// ends. Host code never passes the array's name to a kernel (in host code it is a stand-in, not a
// device address): hipGetSymbolAddress gives each device's own copy, taken once per device on the
// first call there, with that device current.
constexpr size_t kNoAllocBytes = ORPO_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kNoAllocBytes];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

orpo_status scratch_of_current_device(void** out) {
  int dev = -1;
  ORPO_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return ORPO_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    ORPO_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return ORPO_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ORPO_OK;
}

}  // namespace

extern "C" {

orpo_status orpo_head_fwd_noalloc(const orpo_head_desc* desc, const void* h, orpo_weight W,
                                  const int32_t* labels, float* logp, float* lse,
                                  hipStream_t stream) {
  Kind k;
  orpo_status st = check_desc(desc, &k);
  if (st != ORPO_OK) return st;
  if ((st = check_weight(k, W)) != ORPO_OK) return st;
  const FwdPlan p = plan_fwd(desc);
  if (p.ws > kNoAllocBytes) return ORPO_ENOWS;   // the scratch array is too small for this call
  if (desc->M == 0) return ORPO_OK;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != ORPO_OK) return st;
  // Nothing in the workspace needs clearing: the forward kernel zeroes the status word itself and
  // every partial it later reads is written by this call.
  return fwd_impl(desc, k, h, W, nullptr, labels, logp, lse, ws, p.ws, stream);
}

orpo_status orpo_head_fwd_fp8(const orpo_head_desc* desc, const orpo_fp8_operands* q,
                              const int32_t* labels, float* logp, float* lse, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  Kind k;
  orpo_status st = check_desc(desc, &k);
  if (st != ORPO_OK) return st;
  if ((st = check_fp8(desc, k, q)) != ORPO_OK) return st;
  return fwd_impl(desc, k, nullptr, orpo_weight{}, q, labels, logp, lse, ws, ws_bytes, stream);
}

orpo_status orpo_quantize_fp8(const void* x, int64_t rows, int64_t cols, uint8_t* q,
                              uint8_t* exps, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || rows > 4 * int64_t(INT32_MAX)) return ORPO_EINVAL;
  if (rows == 0) return ORPO_OK;
  if (!x || !q || !exps || (uintptr_t)x % 16 || (uintptr_t)q % 8) return ORPO_EINVAL;
  TraceScope ts(ORPO_K_QUANT, 0.0, stream);
  hipLaunchKernelGGL(quant_fp8_kernel, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, stream,
                     (const uint16_t*)x, rows, cols, q, exps);
  return launched();
}

orpo_status orpo_q4_stage(orpo_weight W, int64_t V, int64_t d, void* w_bf16, hipStream_t stream) {
  if (V <= 0 || d <= 0 || d % 64 != 0 || V > INT32_MAX || d > (int64_t(1) << 20)) return ORPO_EINVAL;
  if (!W.w || !W.scales || !W.biases || !w_bf16) return ORPO_EINVAL;
  if ((uintptr_t)W.w % 4 || (uintptr_t)W.scales % 2 || (uintptr_t)W.biases % 2 ||
      (uintptr_t)w_bf16 % 16)
    return ORPO_EINVAL;
  Q4Weight q;
  q.wq = (const uint32_t*)W.w;
  q.scales = (const uint16_t*)W.scales;
  q.biases = (const uint16_t*)W.biases;
  q.V = V;
  q.d = d;
  const int64_t n_words = V * (d / 8);
  // Enough workgroups to keep every CU's loads in flight; the loop strides over the rest.
  const int64_t blocks = std::min<int64_t>(cdiv(n_words, 256 * kQ4StagePer), 256 * 16);
  TraceScope ts(ORPO_K_STAGE, 0.0, stream);
  hipLaunchKernelGGL(q4_stage_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q,
                     (uint16_t*)w_bf16, n_words);
  return launched();
}

static orpo_status loss_impl(int32_t S, int64_t M, int32_t n_pairs, const int32_t* seg_offsets,
                             const float* logp, const int32_t* labels, int64_t V,
                             int32_t ignore_index, double lambda, double* out, float* g, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || M > INT32_MAX || n_pairs < 1 || V <= 0 || V > INT32_MAX) return ORPO_EINVAL;
  if (n_pairs > INT32_MAX / 3) return ORPO_EINVAL;
  if (!seg_offsets || !out || (M > 0 && (!logp || !labels || !g))) return ORPO_EINVAL;
  if (!(lambda == lambda)) return ORPO_EINVAL;
  const size_t need = orpo_loss_workspace_bytes(M, n_pairs);
  if (!ws || ws_bytes < need || (uintptr_t)ws % 256) return ORPO_ENOWS;
  LossArgs a;
  a.M = M;
  a.V = V;
  a.P = n_pairs;
  a.S = S;
  a.off = seg_offsets;
  a.logp = logp;
  a.labels = labels;
  a.ignore_index = ignore_index;
  a.lam = lambda;
  a.out = out;
  a.g = g;
  double* base = (double*)((char*)ws + kHeader);
  const size_t P3 = 3 * size_t(n_pairs);
  a.ell = base;
  a.sum = base + P3;
  a.dl = base + 2 * P3;
  a.cnt = (int64_t*)(base + 3 * P3);
  a.pair = base + 4 * P3;
  a.status = (uint32_t*)ws;
  TraceScope ts(ORPO_K_LOSS, 0.0, stream);
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(1024), 0, stream, a);
  return launched();
}

orpo_status orpo_loss(int64_t M, int32_t n_pairs, const int32_t* seg_offsets, const float* logp,
                      const int32_t* labels, int64_t V, int32_t ignore_index, double lambda,
                      double* out, float* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  return loss_impl(2, M, n_pairs, seg_offsets, logp, labels, V, ignore_index, lambda, out, g, ws,
                   ws_bytes, stream);
}

orpo_status orpo_loss_full(int64_t M, int32_t n_pairs, const int32_t* seg_offsets,
                           const float* logp, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double lambda, double* out, float* g, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  return loss_impl(3, M, n_pairs, seg_offsets, logp, labels, V, ignore_index, lambda, out, g, ws,
                   ws_bytes, stream);
}

size_t orpo_objective_workspace_bytes(int64_t M, int32_t n_spans) {
  if (M < 0 || n_spans < 1) return 0;
  return kHeader + round_up(size_t(n_spans) * 8 * 8, 256);
}

orpo_status orpo_pref_loss(int32_t kind, int64_t M, int32_t n_pairs, const int32_t* seg_offsets,
                           const float* logp, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double beta, double gamma, const double* ref_sums,
                           double* out, float* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (kind < ORPO_PREF_SIMPO || kind > ORPO_PREF_HINGE) return ORPO_EINVAL;
  if (M < 0 || M > INT32_MAX || n_pairs < 1 || n_pairs > INT32_MAX / 2 || V <= 0 || V > INT32_MAX)
    return ORPO_EINVAL;
  if (!seg_offsets || !out || (M > 0 && (!logp || !labels || !g))) return ORPO_EINVAL;
  if (kind == ORPO_PREF_DPO && !ref_sums) return ORPO_EINVAL;
  if (!(beta == beta) || !(gamma == gamma)) return ORPO_EINVAL;
  if (kind == ORPO_PREF_IPO && !(beta > 0.0)) return ORPO_EINVAL;
  if (!ws || ws_bytes < orpo_objective_workspace_bytes(M, 2 * n_pairs) || (uintptr_t)ws % 256)
    return ORPO_ENOWS;
  PrefArgs a;
  a.kind = kind;
  a.M = M;
  a.V = V;
  a.P = n_pairs;
  a.off = seg_offsets;
  a.logp = logp;
  a.labels = labels;
  a.ignore_index = ignore_index;
  a.beta = beta;
  a.gamma = gamma;
  a.ref = ref_sums;
  a.out = out;
  a.g = g;
  double* base = (double*)((char*)ws + kHeader);
  const size_t P = size_t(n_pairs);
  a.val = base;
  a.dv = base + 2 * P;
  a.cnt = (long long*)(base + 4 * P);
  a.pair = base + 6 * P;
  a.status = (uint32_t*)ws;
  TraceScope ts(ORPO_K_LOSS, 0.0, stream);
  hipLaunchKernelGGL(pref_loss_kernel, dim3(1), dim3(1024), 0, stream, a);
  return launched();
}

orpo_status orpo_grpo_loss(int64_t M, int32_t n_seqs, const int32_t* seg_offsets,
                           const float* logp, const float* old_logp, const float* ref_logp,
                           const float* advantages, const int32_t* labels, int64_t V,
                           int32_t ignore_index, double clip_eps, double beta, double* out,
                           float* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || M > INT32_MAX || n_seqs < 1 || V <= 0 || V > INT32_MAX) return ORPO_EINVAL;
  if (!seg_offsets || !out || !advantages) return ORPO_EINVAL;
  if (M > 0 && (!logp || !old_logp || !ref_logp || !labels || !g)) return ORPO_EINVAL;
  if (!(clip_eps >= 0.0) || !(beta == beta)) return ORPO_EINVAL;
  if (!ws || ws_bytes < orpo_objective_workspace_bytes(M, n_seqs) || (uintptr_t)ws % 256)
    return ORPO_ENOWS;
  GrpoArgs a;
  a.M = M;
  a.V = V;
  a.S = n_seqs;
  a.off = seg_offsets;
  a.logp = logp;
  a.old_logp = old_logp;
  a.ref_logp = ref_logp;
  a.adv = advantages;
  a.labels = labels;
  a.ignore_index = ignore_index;
  a.eps = clip_eps;
  a.beta = beta;
  a.out = out;
  a.g = g;
  double* base = (double*)((char*)ws + kHeader);
  const size_t S = size_t(n_seqs);
  a.pg = base;
  a.kl = base + S;
  a.cnt = (long long*)(base + 2 * S);
  a.clipped = (long long*)(base + 3 * S);
  a.status = (uint32_t*)ws;
  TraceScope ts(ORPO_K_LOSS, 0.0, stream);
  hipLaunchKernelGGL(grpo_loss_kernel, dim3(1), dim3(1024), 0, stream, a);
  return launched();
}

}  // extern "C"

namespace {

// The backward of either head (q8: the FP8 head's logit operands for the coefficient recompute).
orpo_status bwd_impl(const orpo_head_desc* desc, Kind k, const void* h, const orpo_weight& W,
                     const orpo_fp8_operands* q8, const int32_t* labels, const float* lse,
                     const float* g, void* dh, float* dW, void* ws, size_t ws_bytes,
                     const void* fwd_ws, hipStream_t stream) {
  orpo_status st;
  if (k == kQ4 && dW) return ORPO_EUNSUPPORTED;
  if ((desc->flags & ORPO_DH_BF16) && k == kF32) return ORPO_EUNSUPPORTED;
  const BwdPlan p = plan_bwd(desc, k);
  if (!bwd_plan_supported(desc, p)) return ORPO_EUNSUPPORTED;
  if (!ws || ws_bytes < p.ws || (uintptr_t)ws % 256) return ORPO_ENOWS;
  if (desc->M == 0) {
    // No token: the weight gradient is zero (overwritten unless accumulating).
    if (dW && !(desc->flags & ORPO_DW_ACCUMULATE)) {
      const int64_t n = desc->V * desc->d;
      const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 65536);
      hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dW, n);
      return launched();
    }
    return ORPO_OK;
  }
  if (!h || !labels || !lse || !g || !dh) return ORPO_EINVAL;

  BwdArgs a{};
  a.h = h;
  a.w = W.w;
  a.q4 = q4_of(desc, W);
  if (q8) {
    a.hq = q8->hq;
    a.wq = q8->wq;
    a.h_exp = q8->h_exp;
    a.w_exp = q8->w_exp;
  }
  a.labels = labels;
  a.lse = lse;
  a.g = g;
  const bool dh_bf16 = (desc->flags & ORPO_DH_BF16) != 0;
  a.dh = dh_bf16 ? nullptr : (float*)dh;
  a.dh16 = dh_bf16 ? (uint16_t*)dh : nullptr;
  a.dh_acc = p.dh_acc_bytes ? (float*)((char*)ws + p.ws - p.dh_acc_bytes) : nullptr;
  a.dW = dW;
  a.M = desc->M;
  a.d = desc->d;
  a.V = desc->V;
  a.BVb = p.BVb;
  a.cap = desc->softcap;
  a.ignore_index = desc->ignore_index;
  a.n_jt = (int)cdiv(desc->d, kTile);
  a.skip_eps = desc->skip_eps;
  a.nsl_v = (int32_t)(p.BVb / 64);
  a.nsl_t = (int32_t)(p.C / 64);
  a.tmax = (a.skip_eps > 0.f && fwd_ws) ? (const float*)((const char*)fwd_ws + plan_fwd(desc).tmax_off)
                                        : nullptr;
  a.n_vtiles = (int32_t)cdiv(desc->V, kTile);
  const bool sc = desc->softcap > 0.f;
  const bool acc_dw = (desc->flags & ORPO_DW_ACCUMULATE) != 0;
  const size_t esize = k == kF32 ? 4 : 2;
  const size_t cbytes = size_t(p.C) * size_t(p.BVb) * esize;
  char* buf[2] = {(char*)ws + kHeader, (char*)ws + kHeader + cbytes};
  uint8_t* flg[2] = {(uint8_t*)ws + kHeader + 2 * cbytes, (uint8_t*)ws + kHeader + 2 * cbytes + p.fl_bytes};
  const size_t fdh_bytes = size_t(p.C / kTile) * size_t(p.BVb / 64) * 4;
  const int64_t n_blocks = cdiv(desc->V, p.BVb);
  const int64_t n_items = cdiv(desc->M, p.C) * n_blocks;
  // Item i = (chunk i / n_blocks, block i % n_blocks); launch i = coefficients of item i + dh/dW of item i-1.
  auto make_item = [&](int64_t i, bool gemm, int split) {
    BwdItem it{};
    if (i < 0 || i >= n_items) return it;   // n_tiles = 0: absent
    const int64_t c = i / n_blocks, blk = i % n_blocks;
    it.c0 = c * p.C;
    it.C_cur = std::min(p.C, desc->M - it.c0);
    it.v0 = blk * p.BVb;
    it.BV_cur = std::min(p.BVb, desc->V - it.v0);
    it.coeff = buf[i % 2];
    it.fdh = p.fl_bytes ? flg[i % 2] : nullptr;
    it.fdw = p.fl_bytes ? flg[i % 2] + fdh_bytes : nullptr;
    it.n_vt = (int)cdiv(it.BV_cur, kTile);
    it.n_tt = (int)cdiv(it.C_cur, kTile);
    it.dh_first = blk == 0;
    it.dh_last = blk == n_blocks - 1;
    it.dw_first = c == 0 && !acc_dw;
    if (gemm) {
      it.dh_split = split;
      it.dh_part = split > 1 ? (float*)((char*)ws + p.part_off) : nullptr;
      it.dh_part_pitch = p.C * desc->d;
      it.n_dh = it.n_tt * a.n_jt * split;
      it.n_tiles = it.n_dh + (dW ? it.n_vt * a.n_jt : 0);
    } else {
      it.n_tiles = it.n_vt * it.n_tt;
    }
    return it;
  };
  for (int64_t i = 0; i <= n_items; ++i) {
    a.cf = make_item(i, false, 1);
    a.gm = make_item(i - 1, true, i < n_items ? p.dh_split : p.dh_split_last);
    const int grid = a.cf.n_tiles + a.gm.n_tiles;
    if (q8) st = sc ? launch_bwd<EBf16, false, true, true>(a, grid, stream) : launch_bwd<EBf16, false, false, true>(a, grid, stream);
    else if (k == kF32) st = sc ? launch_bwd<EF32, false, true>(a, grid, stream) : launch_bwd<EF32, false, false>(a, grid, stream);
    else if (k == kBf16) st = sc ? launch_bwd<EBf16, false, true>(a, grid, stream) : launch_bwd<EBf16, false, false>(a, grid, stream);
    else st = sc ? launch_bwd<EBf16, true, true>(a, grid, stream) : launch_bwd<EBf16, true, false>(a, grid, stream);
    if (st != ORPO_OK) return st;
    if (a.gm.n_tiles > 0 && a.gm.dh_split > 1) {   // the split dh tiles' partials, in split order
      TraceScope ts(ORPO_K_DHSUM, 0.0, stream);
      const int64_t n = a.gm.C_cur * desc->d;
      hipLaunchKernelGGL(dh_reduce_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 2048)),
                         dim3(256), 0, stream, a);
      if ((st = launched()) != ORPO_OK) return st;
    }
  }
  return ORPO_OK;
}

}  // namespace

extern "C" {

orpo_status orpo_head_bwd(const orpo_head_desc* desc, const void* h, orpo_weight W,
                          const int32_t* labels, const float* lse, const float* g, void* dh,
                          float* dW, void* ws, size_t ws_bytes, const void* fwd_ws,
                          hipStream_t stream) {
  Kind k;
  orpo_status st = check_desc(desc, &k);
  if (st != ORPO_OK) return st;
  if ((st = check_weight(k, W)) != ORPO_OK) return st;
  return bwd_impl(desc, k, h, W, nullptr, labels, lse, g, dh, dW, ws, ws_bytes, fwd_ws, stream);
}

orpo_status orpo_head_bwd_fp8(const orpo_head_desc* desc, const orpo_fp8_operands* q,
                              const void* h, orpo_weight W, const int32_t* labels,
                              const float* lse, const float* g, void* dh, float* dW, void* ws,
                              size_t ws_bytes, const void* fwd_ws, hipStream_t stream) {
  Kind k;
  orpo_status st = check_desc(desc, &k);
  if (st != ORPO_OK) return st;
  if ((st = check_weight(k, W)) != ORPO_OK) return st;
  if ((st = check_fp8(desc, k, q)) != ORPO_OK) return st;
  return bwd_impl(desc, k, h, W, q, labels, lse, g, dh, dW, ws, ws_bytes, fwd_ws, stream);
}

orpo_status orpo_set_bwd_tiling(int64_t chunk_tokens, size_t coeff_bytes) {
  if (chunk_tokens < 0 || chunk_tokens % kTile != 0) return ORPO_EINVAL;
  // Bounds that keep every workspace size below 2^54 bytes, so no size product can wrap.
  if (chunk_tokens > (int64_t(1) << 31) || coeff_bytes > (size_t(1) << 40)) return ORPO_EINVAL;
  g_chunk = chunk_tokens ? chunk_tokens : kChunkDefault;
  g_coeff_budget = coeff_bytes;
  return ORPO_OK;
}

orpo_status orpo_trace_enable(int32_t max_launches) {
  if (max_launches < 0) return ORPO_EINVAL;
  for (auto& r : g_trace) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.end);
  }
  g_trace.clear();
  g_trace_used = 0;
  g_trace_on = false;
  for (int32_t i = 0; i < max_launches; ++i) {
    TraceRec r{};
    ORPO_HIP(hipEventCreate(&r.start));
    ORPO_HIP(hipEventCreate(&r.end));
    g_trace.push_back(r);
  }
  g_trace_on = max_launches > 0;
  return ORPO_OK;
}

orpo_status orpo_trace_collect(int32_t kind, int64_t* launches, double* total_ms, double* flops) {
  if (kind < 0 || kind >= ORPO_K_COUNT || !launches || !total_ms || !flops) return ORPO_EINVAL;
  *launches = 0;
  *total_ms = 0.0;
  *flops = 0.0;
  for (size_t i = 0; i < g_trace_used; ++i) {
    const TraceRec& r = g_trace[i];
    if (r.kind != kind) continue;
    ORPO_HIP(hipEventSynchronize(r.end));
    float ms = 0.f;
    ORPO_HIP(hipEventElapsedTime(&ms, r.start, r.end));
    *launches += 1;
    *total_ms += ms;
    *flops += r.flops;
  }
  return ORPO_OK;
}

orpo_status orpo_trace_reset(void) {
  g_trace_used = 0;
  return ORPO_OK;
}

orpo_status orpo_read_status(const void* ws, uint32_t* status_out, hipStream_t stream) {
  if (!ws || !status_out) return ORPO_EINVAL;
  uint32_t v = 0;
  ORPO_HIP(hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream));
  ORPO_HIP(hipStreamSynchronize(stream));
  *status_out = v;
  return ORPO_OK;
}

orpo_status orpo_check(const void* ws, hipStream_t stream) {
  uint32_t v = 0;
  const orpo_status st = orpo_read_status(ws, &v, stream);
  if (st != ORPO_OK) return st;
  return v ? ORPO_EDATA : ORPO_OK;
}

const char* orpo_status_string(int32_t status) {
  switch (status) {
    case ORPO_OK: return "ok";
    case ORPO_EINVAL: return "invalid argument";
    case ORPO_EUNSUPPORTED: return "unsupported shape or format";
    case ORPO_ENOWS: return "workspace missing, misaligned or too small";
    case ORPO_EHIP: return "HIP runtime error";
    case ORPO_EDATA: return "data error reported by the device (see the status word)";
  }
  return "unknown status";
}

int32_t orpo_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
