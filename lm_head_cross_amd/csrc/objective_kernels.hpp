// objective_kernels.hpp — scalar epilogues of the sibling objectives that reuse the head's forward
// (per-token log-probs) and backward (per-token cotangent g). Each runs in one 1024-thread
// workgroup, in float64, with fixed-order reductions (results are bitwise repeatable).
#pragma once
#include "head_kernels.hpp"

namespace orpo {

enum : int32_t { kPrefSimpo = 1, kPrefDpo = 2, kPrefIpo = 3, kPrefHinge = 4 };

// Branch values are length-normalised means for SimPO and IPO, per-sequence sums otherwise.
__device__ __forceinline__ bool pref_mean(int32_t kind) { return kind == kPrefSimpo || kind == kPrefIpo; }

__device__ __forceinline__ double softplus_d(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
__device__ __forceinline__ double sigmoid_d(double x) {
  return x >= 0 ? 1.0 / (1.0 + exp(-x)) : exp(x) / (1.0 + exp(x));
}

struct PrefArgs {
  int32_t kind;           // kPref*
  int64_t M, V;
  int32_t P;
  const int32_t* off;     // [2P+1]: chosen 2p, rejected 2p+1
  const float* logp;
  const int32_t* labels;
  int32_t ignore_index;
  double beta, gamma;
  const double* ref;      // [2P] reference sequence sums (DPO)
  double* out;            // [3 + 2P]: loss, accuracy, margin, v_w[P], v_r[P]
  float* g;
  double* val;            // ws [2P]: per-span value (mean for SimPO, sum for DPO)
  double* dv;             // ws [2P]: dL/dvalue
  long long* cnt;         // ws [2P]
  double* pair;           // ws [3P]: loss term, accuracy bit, margin term
  uint32_t* status;
};

// SimPO (Training — design, §8.3 "Objective variants and data"): per pair
// L = softplus(-beta ((lw - lr) - gamma)) on the length-normalised means. DPO (the post-training
// design's "Stage P1 — DPO"): Delta = beta [(s_w - ref_w) - (s_r - ref_r)] on per-sequence sums,
// L = -log sigma(Delta). IPO and hinge/SLiC (named in the same §8.3 without formulas; read as the
// published losses on the log-ratio margin h = (v_w - ref_w) - (v_r - ref_r), references optional):
// IPO L = (h - 1/(2 beta))^2 on the means, hinge L = max(0, 1 - beta h) on the sums (zero
// gradient at the kink). loss = mean over pairs; g_t = dL/dvalue_s / n_s (means) or dL/dvalue_s
// (sums) for a valid token of span s.
__global__ __launch_bounds__(1024) void pref_loss_kernel(PrefArgs a) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, ns = 2 * a.P;
  const double nan = __builtin_nan("");
  if (check_offsets(a.off, ns, a.M, a.status)) {
    for (int i = tid; i < 3 + ns; i += 1024) a.out[i] = nan;
    for (int64_t t = tid; t < a.M; t += 1024) a.g[t] = nan;
    return;
  }
  for (int s = w; s < ns; s += 16) {
    double sum;
    long long n;
    span_sum(a.off, s, a.logp, a.labels, a.ignore_index, a.V, &sum, &n);
    if (l == 0) {
      a.cnt[s] = n;
      a.val[s] = n == 0 ? nan : (pref_mean(a.kind) ? sum / (double)n : sum);
      if (n == 0) atomicOr(a.status, kStatusEmptyBranch);
    }
  }
  __syncthreads();
  for (int p = tid; p < a.P; p += 1024) {
    const double vw = a.val[2 * p], vr = a.val[2 * p + 1];
    double lp, d, margin, acc;
    if (a.kind == kPrefSimpo) {
      const double u = a.beta * ((vw - vr) - a.gamma);
      lp = softplus_d(-u);
      d = -a.beta * sigmoid_d(-u) / (double)a.P;
      margin = vw - vr;
      acc = vw > vr ? 1.0 : 0.0;
    } else {
      const double rw = a.ref ? a.ref[2 * p] : 0.0, rr = a.ref ? a.ref[2 * p + 1] : 0.0;
      const double hm = (vw - rw) - (vr - rr);
      if (a.kind == kPrefDpo) {
        const double u = a.beta * hm;
        lp = softplus_d(-u);
        d = -a.beta * sigmoid_d(-u) / (double)a.P;
        margin = u;
      } else if (a.kind == kPrefIpo) {
        const double e = hm - 1.0 / (2.0 * a.beta);
        lp = e * e;
        d = 2.0 * e / (double)a.P;
        margin = hm;
      } else {
        const double u = 1.0 - a.beta * hm;
        lp = u > 0 ? u : 0.0;
        d = u > 0 ? -a.beta / (double)a.P : 0.0;
        margin = hm;
      }
      acc = hm > 0 ? 1.0 : 0.0;
    }
    a.dv[2 * p] = d;
    a.dv[2 * p + 1] = -d;
    a.pair[p] = lp;
    a.pair[a.P + p] = acc;
    a.pair[2 * a.P + p] = margin;
    a.out[3 + p] = vw;
    a.out[3 + a.P + p] = vr;
  }
  __syncthreads();
  if (w == 0) {
    const double lo = wave_sum<double>(a.P, [&](int p) { return a.pair[p]; });
    const double ac = wave_sum<double>(a.P, [&](int p) { return a.pair[a.P + p]; });
    const double mg = wave_sum<double>(a.P, [&](int p) { return a.pair[2 * a.P + p]; });
    if (l == 0) {
      a.out[0] = lo / (double)a.P;
      a.out[1] = ac / (double)a.P;
      a.out[2] = mg / (double)a.P;
    }
  }
  fill_g_by_span(a.off, ns, a.M, a.labels, a.ignore_index, a.V, a.g, [&](int s) {
    const float gs = a.cnt[s] > 0 ? (float)(pref_mean(a.kind) ? a.dv[s] / (double)a.cnt[s] : a.dv[s])
                                  : 0.f;
    return [gs](int64_t) { return gs; };
  });
}

struct GrpoArgs {
  int64_t M, V;
  int32_t S;              // completions
  const int32_t* off;     // [S+1]
  const float* logp;
  const float* old_logp;
  const float* ref_logp;
  const float* adv;       // [S]
  const int32_t* labels;
  int32_t ignore_index;
  double eps, beta;
  double* out;            // [4]: loss, pg, kl, clip fraction
  float* g;
  double* pg;             // ws [S] per-completion mean of the policy-gradient term
  double* kl;             // ws [S] per-completion mean k3
  long long* cnt;         // ws [S]
  long long* clipped;     // ws [S]
  uint32_t* status;
};

// One token's policy-gradient term, k3 term and their derivatives w.r.t. logp (the post-training
// design's "Stage P3 — GRPO", (d)): rho = exp(logp - old); pg = -min(rho A, clip(rho, 1-eps, 1+eps) A);
// k3 = exp(ref - logp) - (ref - logp) - 1. d pg / d logp = -A rho where the unclipped term is the
// minimum (ties included), else 0; d k3 / d logp = 1 - exp(ref - logp).
struct GrpoToken {
  double pg, k3, dpg, dk3;
  bool clipped;
};
__device__ __forceinline__ GrpoToken grpo_token(double lp, double old, double ref, double A, double eps) {
  GrpoToken r;
  const double rho = exp(lp - old);
  const double un = rho * A, cl = fmin(fmax(rho, 1.0 - eps), 1.0 + eps) * A;
  r.clipped = un > cl;
  r.pg = -(r.clipped ? cl : un);
  r.dpg = r.clipped ? 0.0 : -A * rho;
  const double d = ref - lp, ed = exp(d);
  r.k3 = ed - d - 1.0;
  r.dk3 = 1.0 - ed;
  return r;
}

// loss = mean over completions of (mean over the completion's valid tokens of pg + beta k3);
// g_t = (dpg + beta dk3) / (n_s S).
__global__ __launch_bounds__(1024) void grpo_loss_kernel(GrpoArgs a) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const double nan = __builtin_nan("");
  if (check_offsets(a.off, a.S, a.M, a.status)) {
    for (int i = tid; i < 4; i += 1024) a.out[i] = nan;
    for (int64_t t = tid; t < a.M; t += 1024) a.g[t] = nan;
    return;
  }
  for (int s = w; s < a.S; s += 16) {
    double pg = 0.0, kl = 0.0;
    long long n = 0, c = 0;
    const double A = (double)a.adv[s];
    for (int64_t t = a.off[s] + l; t < a.off[s + 1]; t += 64) {
      const int y = a.labels[t];
      if (y != a.ignore_index && y >= 0 && (int64_t)y < a.V) {
        const GrpoToken r = grpo_token(a.logp[t], a.old_logp[t], a.ref_logp[t], A, a.eps);
        pg += r.pg;
        kl += r.k3;
        ++n;
        c += r.clipped;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      pg += __shfl_xor(pg, o);
      kl += __shfl_xor(kl, o);
      n += __shfl_xor(n, o);
      c += __shfl_xor(c, o);
    }
    if (l == 0) {
      a.cnt[s] = n;
      a.clipped[s] = c;
      a.pg[s] = n ? pg / (double)n : nan;
      a.kl[s] = n ? kl / (double)n : nan;
      if (n == 0) atomicOr(a.status, kStatusEmptyBranch);
    }
  }
  __syncthreads();
  if (w == 0) {
    const double pg = wave_sum<double>(a.S, [&](int s) { return a.pg[s]; }) / (double)a.S;
    const double kl = wave_sum<double>(a.S, [&](int s) { return a.kl[s]; }) / (double)a.S;
    const long long n = wave_sum<long long>(a.S, [&](int s) { return (long long)a.cnt[s]; });
    const long long c = wave_sum<long long>(a.S, [&](int s) { return (long long)a.clipped[s]; });
    if (l == 0) {
      a.out[0] = pg + a.beta * kl;
      a.out[1] = pg;
      a.out[2] = kl;
      a.out[3] = n ? (double)c / (double)n : nan;
    }
  }
  fill_g_by_span(a.off, a.S, a.M, a.labels, a.ignore_index, a.V, a.g, [&](int s) {
    const double adv = (double)a.adv[s], den = (double)a.cnt[s] * (double)a.S;
    return [&a, adv, den](int64_t t) {
      const GrpoToken r = grpo_token(a.logp[t], a.old_logp[t], a.ref_logp[t], adv, a.eps);
      return (float)((r.dpg + a.beta * r.dk3) / den);
    };
  });
}

}  // namespace orpo
