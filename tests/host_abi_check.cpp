// Host-side sweep of the C ABI's argument checking, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only and run without a GPU.
//
// Every call below must return before it reaches the HIP runtime: either the arguments are
// rejected, or the workspace is one byte short of the size the library itself reported. The sweep
// covers extreme sizes (negative, zero, 2^31 - 1, 2^63 - 1), every storage format pair, NaN and
// infinite scalars, unknown flags, and the backward tiling knob at its bounds, and checks that
//   - workspace sizes are multiples of 256 and 0 exactly where the entry point refuses the call,
//   - an entry point refuses with EINVAL / EUNSUPPORTED where the size query says 0, and asks for
//     more workspace (ENOWS) otherwise,
//   - no size arithmetic overflows (UBSan) and no host memory is touched out of bounds (ASan).
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "orpo_head.h"

namespace {

long g_fails = 0;
long g_checks = 0;

#define EXPECT(cond)                                                                   \
  do {                                                                                 \
    ++g_checks;                                                                        \
    if (!(cond)) {                                                                     \
      if (g_fails < 20) std::printf("FAIL line %d: %s\n", __LINE__, #cond);            \
      ++g_fails;                                                                       \
    }                                                                                  \
  } while (0)

// Stand-in device pointers: never dereferenced, since no call below may launch a kernel.
void* fake(uintptr_t v) { return reinterpret_cast<void*>(v); }
const uintptr_t kPtr = 4096;       // 256-aligned
const uintptr_t kWs = 1 << 20;     // 256-aligned workspace address

bool refused(orpo_status st) { return st == ORPO_EINVAL || st == ORPO_EUNSUPPORTED; }

orpo_weight weight_for(int32_t w_fmt) {
  orpo_weight w{};
  w.w = fake(kPtr);
  if (w_fmt == ORPO_Q4G64) {
    w.scales = fake(kPtr);
    w.biases = fake(kPtr);
  }
  return w;
}

void check_head(const orpo_head_desc& d) {
  const size_t fw = orpo_head_fwd_workspace_bytes(&d);
  const size_t bw = orpo_head_bwd_workspace_bytes(&d);
  EXPECT(fw % 256 == 0);
  EXPECT(bw % 256 == 0);
  if (fw != 0) EXPECT(fw >= 256);
  if (bw != 0) EXPECT(bw >= 256 && fw != 0);   // a backward needs a valid forward

  const orpo_weight w = weight_for(d.w_fmt);
  void* p = fake(kPtr);
  orpo_status st = orpo_head_fwd(&d, p, w, (const int32_t*)p, (float*)p, (float*)p, fake(kWs),
                                 fw ? fw - 1 : std::numeric_limits<size_t>::max(), nullptr);
  if (fw == 0) EXPECT(refused(st));
  else EXPECT(st == ORPO_ENOWS);

  for (int with_dw = 0; with_dw < 2; ++with_dw) {
    float* dW = with_dw ? (float*)p : nullptr;
    st = orpo_head_bwd(&d, p, w, (const int32_t*)p, (const float*)p, (const float*)p, p, dW,
                       fake(kWs), bw ? bw - 1 : std::numeric_limits<size_t>::max(), nullptr,
                       nullptr);
    if (bw == 0) EXPECT(refused(st));
    else if (with_dw && d.w_fmt == ORPO_Q4G64) EXPECT(st == ORPO_EUNSUPPORTED);   // frozen head
    else EXPECT(st == ORPO_ENOWS);
  }
  // The FP8 head: the same sizes; refused unless the head is bf16 with d a multiple of 128, and
  // not with both a softcap above 40 and the coefficient filter.
  const orpo_fp8_operands q8 = {(const uint8_t*)p, (const uint8_t*)p, (const uint8_t*)p,
                                (const uint8_t*)p};
  const bool fp8_ok = d.h_fmt == ORPO_BF16 && d.w_fmt == ORPO_BF16 && d.d % 128 == 0 &&
                      !(d.softcap > 40.f && d.skip_eps > 0.f);
  st = orpo_head_fwd_fp8(&d, &q8, (const int32_t*)p, (float*)p, (float*)p, fake(kWs),
                         fw ? fw - 1 : std::numeric_limits<size_t>::max(), nullptr);
  if (fw == 0) EXPECT(refused(st));
  else EXPECT(st == (fp8_ok ? ORPO_ENOWS : ORPO_EUNSUPPORTED));
  EXPECT(orpo_head_fwd_fp8(&d, nullptr, (const int32_t*)p, (float*)p, (float*)p, fake(kWs),
                           std::numeric_limits<size_t>::max(), nullptr) != ORPO_OK);
  st = orpo_head_bwd_fp8(&d, &q8, p, w, (const int32_t*)p, (const float*)p, (const float*)p, p,
                         (float*)p, fake(kWs), bw ? bw - 1 : std::numeric_limits<size_t>::max(),
                         nullptr, nullptr);
  if (bw == 0) EXPECT(refused(st));
  else if (!fp8_ok) EXPECT(st == ORPO_EUNSUPPORTED);
  else EXPECT(st == ORPO_ENOWS);
  // A misaligned workspace of any size is refused as ENOWS once the descriptor is valid.
  st = orpo_head_fwd(&d, p, w, (const int32_t*)p, (float*)p, (float*)p, fake(kWs + 64),
                     std::numeric_limits<size_t>::max(), nullptr);
  if (fw == 0) EXPECT(refused(st));
  else EXPECT(st == ORPO_ENOWS);
}

void sweep_head() {
  const int64_t I32 = std::numeric_limits<int32_t>::max();
  const int64_t I64 = std::numeric_limits<int64_t>::max();
  const float inf = std::numeric_limits<float>::infinity();
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const int64_t Ms[] = {-1, 0, 1, 255, 256, 8192, 32768, I32, I32 + 1, I64};
  const int64_t ds[] = {-64, 0, 32, 64, 2560, int64_t(1) << 20, (int64_t(1) << 20) + 64, I64};
  const int64_t Vs[] = {-1, 0, 1, 257, 262144, int64_t(1) << 22, I32, I32 + 1, I64};
  const int32_t fmts[] = {-1, ORPO_F32, ORPO_BF16, ORPO_Q4G64, 3};
  const float caps[] = {0.f, -1.f, 30.f, 40.f, 40.5f, 1024.f, 1024.5f, inf, -inf, nan};
  const uint32_t flags[] = {0u, ORPO_DW_ACCUMULATE, ORPO_DH_BF16, ORPO_DW_ACCUMULATE | ORPO_DH_BF16, 4u,
                            0x80000000u};
  const float eps[] = {0.f, 1e-5f, -1.f, inf, nan};
  orpo_head_desc d{};
  d.ignore_index = -100;
  for (int64_t M : Ms)
    for (int64_t dd : ds)
      for (int64_t V : Vs)
        for (int32_t hf : fmts)
          for (int32_t wf : fmts)
            for (float cap : caps)
              for (uint32_t fl : flags)
                for (float e : eps) {
                  d.M = M;
                  d.d = dd;
                  d.V = V;
                  d.h_fmt = hf;
                  d.w_fmt = wf;
                  d.softcap = cap;
                  d.flags = fl;
                  d.skip_eps = e;
                  check_head(d);
                }
}

void sweep_tiling() {
  const int64_t I64 = std::numeric_limits<int64_t>::max();
  const size_t SMAX = std::numeric_limits<size_t>::max();
  const int64_t chunks[] = {-256, 0, 100, 256, 8192, int64_t(1) << 31, (int64_t(1) << 31) + 256,
                            I64 - I64 % 256};
  const size_t budgets[] = {0, 1, size_t(1) << 28, size_t(1) << 40, (size_t(1) << 40) + 1, SMAX};
  orpo_head_desc d{};
  d.d = 1 << 20;
  d.V = std::numeric_limits<int32_t>::max();
  d.h_fmt = ORPO_BF16;
  d.w_fmt = ORPO_BF16;
  d.softcap = 30.f;
  d.ignore_index = -100;
  for (int64_t c : chunks)
    for (size_t b : budgets) {
      const orpo_status st = orpo_set_bwd_tiling(c, b);
      const bool ok = c >= 0 && c % 256 == 0 && c <= (int64_t(1) << 31) && b <= (size_t(1) << 40);
      EXPECT(st == (ok ? ORPO_OK : ORPO_EINVAL));
      for (int64_t M : {int64_t(1), int64_t(300000), int64_t(std::numeric_limits<int32_t>::max())})
        for (uint32_t fl : {0u, uint32_t(ORPO_DH_BF16)})
          for (float e : {0.f, 1e-5f}) {
            d.M = M;
            d.flags = fl;
            d.skip_eps = e;
            const size_t ws = orpo_head_bwd_workspace_bytes(&d);
            EXPECT(ws % 256 == 0);
            EXPECT(ws < (size_t(1) << 54));
            if (e == 0.f) EXPECT(ws >= 256);   // the exact backward has no tiling limit
            check_head(d);
          }
    }
  EXPECT(orpo_set_bwd_tiling(0, 0) == ORPO_OK);
}

void sweep_losses() {
  const int64_t I32 = std::numeric_limits<int32_t>::max();
  const int64_t I64 = std::numeric_limits<int64_t>::max();
  const double dnan = std::numeric_limits<double>::quiet_NaN();
  const double dinf = std::numeric_limits<double>::infinity();
  const int64_t Ms[] = {-1, 0, 1, 8192, I32, I32 + 1, I64};
  const int32_t ns[] = {-1, 0, 1, 2, int32_t(I32 / 3), int32_t(I32 / 3 + 1), int32_t(I32 / 2 + 1),
                        int32_t(I32)};
  const int64_t Vs[] = {-1, 0, 1, 262144, I32 + 1};
  const double scalars[] = {0.1, 0.0, -1.0, dnan, dinf};
  void* p = fake(kPtr);
  const int32_t* ip = (const int32_t*)p;
  const float* fp = (const float*)p;
  const size_t SMAX = std::numeric_limits<size_t>::max();
  for (int64_t M : Ms)
    for (int32_t n : ns)
      for (int64_t V : Vs)
        for (double s : scalars) {
          const size_t lw = orpo_loss_workspace_bytes(M, n);
          EXPECT(lw % 256 == 0);
          const orpo_status a = orpo_loss(M, n, ip, fp, ip, V, -100, s, (double*)p, (float*)p,
                                          fake(kWs), lw ? lw - 1 : SMAX, nullptr);
          const orpo_status b = orpo_loss_full(M, n, ip, fp, ip, V, -100, s, (double*)p, (float*)p,
                                               fake(kWs), lw ? lw - 1 : SMAX, nullptr);
          EXPECT(a == ORPO_EINVAL || (lw != 0 && a == ORPO_ENOWS));
          EXPECT(b == a);
          const size_t ow = orpo_objective_workspace_bytes(M, n);
          EXPECT(ow % 256 == 0);
          for (int32_t kind = -1; kind <= 6; ++kind)
            for (int with_ref = 0; with_ref < 2; ++with_ref) {
              const size_t pw = orpo_objective_workspace_bytes(M, n > I32 / 2 ? 0 : 2 * n);
              const orpo_status c = orpo_pref_loss(
                  kind, M, n, ip, fp, ip, V, -100, s, 0.5, with_ref ? (const double*)p : nullptr,
                  (double*)p, (float*)p, fake(kWs), pw ? pw - 1 : SMAX, nullptr);
              EXPECT(c == ORPO_EINVAL || (pw != 0 && c == ORPO_ENOWS));
              if (kind < ORPO_PREF_SIMPO || kind > ORPO_PREF_HINGE) EXPECT(c == ORPO_EINVAL);
              if (kind == ORPO_PREF_DPO && !with_ref) EXPECT(c == ORPO_EINVAL);
              if (kind == ORPO_PREF_IPO && !(s > 0.0)) EXPECT(c == ORPO_EINVAL);
            }
          const orpo_status g = orpo_grpo_loss(M, n, ip, fp, fp, fp, fp, ip, V, -100, s, 0.04,
                                               (double*)p, (float*)p, fake(kWs), ow ? ow - 1 : SMAX,
                                               nullptr);
          EXPECT(g == ORPO_EINVAL || (ow != 0 && g == ORPO_ENOWS));
          if (!(s >= 0.0)) EXPECT(g == ORPO_EINVAL);   // the clip range
        }
}

void sweep_quantize() {
  const int64_t I64 = std::numeric_limits<int64_t>::max();
  for (int64_t rows : {int64_t(-1), int64_t(0), int64_t(1), int64_t(1) << 33, I64})
    for (int64_t cols : {int64_t(-8), int64_t(0), int64_t(4), int64_t(8), int64_t(2560), I64})
      for (uintptr_t xo : {uintptr_t(0), uintptr_t(8)})
        for (uintptr_t qo : {uintptr_t(0), uintptr_t(4)}) {
          const bool shape_ok = rows >= 0 && cols > 0 && cols % 8 == 0 && rows <= 4 * int64_t(INT32_MAX);
          if (shape_ok && rows > 0 && !xo && !qo) continue;   // valid: it would launch
          const orpo_status st = orpo_quantize_fp8(fake(kPtr + xo), rows, cols,
                                                   (uint8_t*)fake(kPtr + qo), (uint8_t*)fake(kPtr),
                                                   nullptr);
          if (!shape_ok) EXPECT(st == ORPO_EINVAL);
          else if (rows == 0) EXPECT(st == ORPO_OK);
          else EXPECT(st == ORPO_EINVAL);                    // misaligned x or q
        }
}

void check_misc() {
  for (int64_t s : {int64_t(std::numeric_limits<int32_t>::min()), int64_t(-5), int64_t(-4),
                    int64_t(-1), int64_t(0), int64_t(1), int64_t(std::numeric_limits<int32_t>::max())})
    EXPECT(orpo_status_string(int32_t(s)) != nullptr);
  int64_t launches = -1;
  double ms = -1, flops = -1;
  EXPECT(orpo_trace_enable(-1) == ORPO_EINVAL);
  EXPECT(orpo_trace_enable(0) == ORPO_OK);   // disables: no event to create
  EXPECT(orpo_trace_reset() == ORPO_OK);
  EXPECT(orpo_trace_collect(-1, &launches, &ms, &flops) == ORPO_EINVAL);
  EXPECT(orpo_trace_collect(0, nullptr, &ms, &flops) == ORPO_EINVAL);
  EXPECT(orpo_trace_collect(0, &launches, &ms, &flops) == ORPO_OK);
  EXPECT(launches == 0 && ms == 0.0 && flops == 0.0);
  EXPECT(orpo_trace_collect(1 << 20, &launches, &ms, &flops) == ORPO_EINVAL);
  uint32_t status = 0;
  EXPECT(orpo_read_status(nullptr, &status, nullptr) == ORPO_EINVAL);
  EXPECT(orpo_read_status(fake(kWs), nullptr, nullptr) == ORPO_EINVAL);
  EXPECT(orpo_head_fwd_workspace_bytes(nullptr) == 0);
  EXPECT(orpo_head_bwd_workspace_bytes(nullptr) == 0);
}

}  // namespace

int main() {
  sweep_head();
  sweep_tiling();
  sweep_losses();
  sweep_quantize();
  check_misc();
  std::printf("%s: %ld checks, %ld failures\n", g_fails ? "FAILED" : "ok", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
