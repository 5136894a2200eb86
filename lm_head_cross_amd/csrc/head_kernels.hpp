// head_kernels.hpp — the flash-CCE ORPO head kernels for gfx950.
//
//   quant_fp8_kernel: bf16 rows -> FP8 E4M3 codes with one power-of-two (E8M0) scale per row, for
//                   the low-precision logit operands.
//   q4_stage_kernel: a 4-bit head -> bf16 rows, the tiled loops' own dequantisation done once.
//   fwd_kernel    : raw = W . h^T tile by tile (MFMA), softcap, online softmax per token over the
//                   workgroup's vocabulary split, label-logit capture -> per-split (max, sum) partials.
//   merge_kernel  : partials of all splits -> lse, logp = z[y] - lse (merge_wide_kernel: the
//                   same with one wave per token, for the many splits of a small M).
//   loss_kernel   : segmented per-branch means (f64), scalar ORPO epilogue (f64), cotangent g.
//   bwd_kernel    : one launch of the backward pipeline: coefficient tiles (recompute a logit tile,
//                   coeff = g (onehot - softmax) sech^2) of one (token chunk, vocabulary block) item
//                   and the dh (+)= coeff . W_blk and dW_blk (+)= coeff^T . h_chunk tiles of the
//                   previous item.
//
// Sources: "Training — design" §1 "The objective" and §5.1 "The head"; its older revision "ORPO
// training — design", "Memory & speed optimization", lever 1 and the "Implementation spec — fused
// linear-CE log-prob head" (online softmax over vocabulary tiles, O(M) saved state, recompute in
// the backward); "Steel flash-CCE — handoff", "The architecture" (per-split partials and their
// merge) and Glossary D "The epilogue" (softcap, online softmax, target capture, softmax-onehot
// coefficient). The (max, sum) running state and every gradient accumulation stay in fp32, as the
// older revision's vocab-blocked head found necessary.
#pragma once
#include <type_traits>

#include "gemm_core.hpp"

namespace orpo {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kStatusBadLabel = 1u, kStatusEmptyBranch = 2u, kStatusBadOffsets = 4u;
constexpr int kMaxKSteps = 8192;   // K steps a dh / dW tile can list under the coefficient filter

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float log2_(float x) { return __builtin_amdgcn_logf(x); }

// Softcap in the log2 domain. With E = 2^(raw * 2 log2e / cap) = e^(2 raw / cap) and
// r = 1 / (E + 1): tanh(raw / cap) = 1 - 2r, so z = cap - 2 cap r and (z - cap) log2e = -2 cap log2e r,
// and sech^2(raw / cap) = 1 - tanh^2 = 4 r (1 - r).
struct Softcap {
  float cap, c1, kz;
  __device__ Softcap(float c) : cap(c), c1(2.f * kLog2e / c), kz(-2.f * c * kLog2e) {}
  __device__ __forceinline__ float r_of(float raw) const { return rcp_(exp2_(raw * c1) + 1.f); }
};

// ------------------------------------------------------------------------------------------
// FP8 E4M3 row quantisation (the low-precision logit operands; "Training — design", §8.1 "Deferred
// performance levers", the W4A16 head GEMM item: half-width operands for the logit GEMM, fp32
// accumulation). Each
// row gets the smallest power-of-two scale 2^e with max|x| <= 448 2^e (e >= -127; e = 0 for a zero
// row), stored as the E8M0 byte e + 127, and every element the E4M3 code nearest to x 2^-e, ties to
// the even code, the sign kept on zero. Codes: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
// bits; S.1111.111 is NaN and never produced (|x 2^-e| <= 448 = S.1111.110).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int fp8_row_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = __builtin_frexpf(amax, &k);     // amax = m 2^k, m in [0.5, 1); 448 = 0.875 2^9
  return max(m <= 0.875f ? k - 9 : k - 8, -127);
}

__device__ __forceinline__ uint32_t e4m3_code(float y) {   // |y| <= 448
  const float a = fabsf(y);
  uint32_t c;
  if (a < 0x1p-6f) {
    c = (uint32_t)__builtin_rintf(a * 0x1p9f);     // subnormal grid n 2^-9; n = 8 is code 8 = 2^-6
  } else {
    int k;
    const float m = __builtin_frexpf(a, &k);       // a = (2m) 2^(k-1): exponent field k - 1 + 7
    c = (uint32_t)((k + 6) << 3) + (uint32_t)__builtin_rintf((2.f * m - 1.f) * 8.f);   // carry ok
  }
  return c | ((__float_as_uint(y) >> 31) << 7);
}

// The codes of 8 consecutive bf16 values (one 16-byte load) at row exponent e.
__device__ __forceinline__ u32x2 e4m3_codes8(const u32x4& v, int e) {
  u32x2 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = e4m3_code(__builtin_ldexpf(bf16_bits_to_f32(v[i] & 0xFFFFu), -e));
    const uint32_t hi = e4m3_code(__builtin_ldexpf(bf16_bits_to_f32(v[i] >> 16), -e));
    const uint32_t pair = lo | (hi << 8);
    if (i & 1) out[i >> 1] |= pair << 16;
    else out[i >> 1] = pair;
  }
  return out;
}

__device__ __forceinline__ float amax8(float m, const u32x4& v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[i] & 0xFFFFu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(v[i] >> 16)));
  }
  return m;
}

// One wave per row: the row maximum, then the codes (8 per lane and iteration). Rows of up to
// kQuantHeld x 512 values are read once and held in registers between the two passes; longer rows
// are read twice. cols is a multiple of 8; x rows 16-byte and q rows 8-byte aligned.
constexpr int kQuantHeld = 8;
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                        uint8_t* q, uint8_t* exps) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= rows) return;
  const uint16_t* xr = x + r * cols;
  uint8_t* qr = q + r * cols;
  float amax = 0.f;
  if (cols <= kQuantHeld * 512) {
    u32x4 v[kQuantHeld];
#pragma unroll
    for (int i = 0; i < kQuantHeld; ++i) {
      const int64_t c = (int64_t)l * 8 + i * 512;
      v[i] = c < cols ? *(const u32x4*)(xr + c) : u32x4{0u, 0u, 0u, 0u};
      amax = amax8(amax, v[i]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const int e = fp8_row_exponent(amax);
#pragma unroll
    for (int i = 0; i < kQuantHeld; ++i) {
      const int64_t c = (int64_t)l * 8 + i * 512;
      if (c < cols) *(u32x2*)(qr + c) = e4m3_codes8(v[i], e);
    }
    if (l == 0) exps[r] = (uint8_t)(e + 127);
    return;
  }
  for (int64_t c = (int64_t)l * 8; c < cols; c += 512) amax = amax8(amax, *(const u32x4*)(xr + c));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int e = fp8_row_exponent(amax);
  for (int64_t c = (int64_t)l * 8; c < cols; c += 512) *(u32x2*)(qr + c) = e4m3_codes8(*(const u32x4*)(xr + c), e);
  if (l == 0) exps[r] = (uint8_t)(e + 127);
}

// A 4-bit head dequantised to bf16 rows in HBM: each lane takes one packed word (8 codes) and
// stores its 16 bytes, so a wave's store covers 1 KB of contiguous output; kQ4StagePer words per
// lane and iteration are loaded before any is converted. The arithmetic is dequant_word's, the
// one the tiled loops apply in LDS (fp32 scale * q + bias, rounded to nearest even), so the
// staged rows equal what those loops would stage, bit for bit. d % 64 == 0: the 8 words of a
// group lie in one row, and word j's group is j / 8 of the flattened [V, d / 64] scales.
constexpr int kQ4StagePer = 4;
__global__ __launch_bounds__(256) void q4_stage_kernel(Q4Weight W, uint16_t* out, int64_t n_words) {
  const int64_t stride = (int64_t)gridDim.x * 256 * kQ4StagePer;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kQ4StagePer + threadIdx.x; base < n_words;
       base += stride) {
    uint32_t q[kQ4StagePer];
    uint16_t sb[kQ4StagePer], bb[kQ4StagePer];
#pragma unroll
    for (int i = 0; i < kQ4StagePer; ++i) {
      const int64_t j = base + i * 256;
      const int64_t jj = j < n_words ? j : 0;
      q[i] = W.wq[jj];
      sb[i] = W.scales[jj >> 3];
      bb[i] = W.biases[jj >> 3];
    }
#pragma unroll
    for (int i = 0; i < kQ4StagePer; ++i) {
      const int64_t j = base + i * 256;
      if (j < n_words)
        *(u32x4*)(out + j * 8) = dequant_word(q[i], bf16_bits_to_f32(sb[i]), bf16_bits_to_f32(bb[i]));
    }
  }
}

// E8M0 exponent bytes of rows r0 + lane_row + 32 i (i < N) packed little-endian, the MFMA's
// per-block scale word (r0 uniform, rows >= 1); rows past `rows` get 127 (2^0: their operand
// data is zero) and read row rows - 1 instead, so every load stays in bounds. 32-bit lane
// offsets keep the live state small.
template <int N>
__device__ __forceinline__ int32_t pack_row_exps(const uint8_t* e, int64_t r0, int lane_row,
                                                 int64_t rows) {
  const uint8_t* base = e + r0;
  const int left = (int)min<int64_t>(rows - r0, 1 << 30);
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int rr = lane_row + 32 * i;
    const uint32_t b = base[rr < left ? rr : left - 1];
    v |= (rr < left ? b : 127u) << (8 * i);
  }
  return (int32_t)v;
}

// ------------------------------------------------------------------------------------------
// Forward
// ------------------------------------------------------------------------------------------
struct FwdArgs {
  const void* h;          // [M, d] (FP8 codes for EFp8)
  const void* w;          // [V, d] dense (FP8 codes for EFp8), or Q4Weight below
  Q4Weight q4;
  const uint8_t* h_exp;   // EFp8: E8M0 row exponents of h [M] and W [V]
  const uint8_t* w_exp;
  const int32_t* labels;  // [M]
  float* logp;            // [M]: receives z[y] here, finished by merge_kernel
  float2* part;           // [nblk, M] (max in log2 units, sum of 2^(u - max))
  float* tmax;            // [n_tb][n_vtiles][8]: per wave, max raw logit of its part of the tile
  uint32_t* status;
  int64_t M, d, V;
  float cap;
  int32_t ignore_index;
  int32_t n_tb, nblk, tiles_per_split, n_vtiles;
};

// Softmax reference of the forward. kSoftcapFixed: every z <= cap, so the sum is taken against
// the fixed reference cap (no max pass, no rescaling); its smallest term 2^(-2 cap log2 e) stays a
// normal float only for cap <= kFixedRefMaxCap. kSoftcapRunMax: larger softcaps keep a running
// maximum, as without a softcap.
enum FwdMode { kNoSoftcap = 0, kSoftcapFixed = 1, kSoftcapRunMax = 2 };
constexpr float kFixedRefMaxCap = 40.f;

// TMAX: the variant that also records each wave's largest raw logit per tile (the backward's
// coefficient filter uses them to skip whole cold coefficient tiles).
template <class E, bool Q4, int MODE, bool TMAX>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  constexpr bool SOFTCAP = MODE != kNoSoftcap;
  constexpr bool kRunMax = MODE != kSoftcapFixed;
  ORPO_DECLARE_SMEM(smem);
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 2, wn = w & 3;
  const int tb = blockIdx.x % a.n_tb, split = blockIdx.x / a.n_tb;
  const int tile0 = split * a.tiles_per_split;
  const int n_tiles = min(a.tiles_per_split, a.n_vtiles - tile0);
  if (blockIdx.x == 0 && tid == 0) *a.status = 0u;
  const int64_t t0 = (int64_t)tb * kTile;
  const int64_t row_bytes = a.d * E::kSize;

  // The token of accumulator column block nb, recomputed where needed rather than held (as two
  // 64-bit values) across the K loop. The 4-bit loop, with its dequantisation registers, needs
  // the column made opaque to keep the compiler from hoisting the sum out of the loop.
  auto tok_of = [&](int nb) {
    int n = acc_n(wn, nb, l);
    if constexpr (Q4) asm("" : "+v"(n));
    return t0 + n;
  };
  int y[2];
  float m[2], s[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t tok = tok_of(nb);
    // -1 marks "no capture": rows past M and ignored tokens (ignore_index may be any value).
    const int lab = tok < a.M ? a.labels[tok] : -1;
    y[nb] = lab == a.ignore_index ? -1 : lab;
    m[nb] = kRunMax ? kNegInf : a.cap * kLog2e;   // fixed reference: every z <= cap
    s[nb] = 0.f;
  }
  const Softcap sc(SOFTCAP ? a.cap : 1.f);

  typedef typename std::conditional<Q4, Q4K2, DmaKS<E::kSwzShift, E::kSwzK>>::type LoaderA;
  LoaderA la;
  DmaKS<E::kSwzShift, E::kSwzK> lb;
  if constexpr (Q4) la.init(a.q4); else la.init(a.w, row_bytes, a.V);
  lb.init(a.h, row_bytes, a.M);
  const int nk = (int)(a.d / E::kBK);
  // Dense weights: both operands by direct loads. 4-bit weights (gemm_run_q4k): the words of a
  // step by register loads into one of two sets (rows past V read row 0 and are zeroed), the hidden
  // states by direct loads.
  auto issue = [&](int tile, int ks, char* sa, char* sb) {
    if constexpr (!Q4) la.issue((int64_t)(tile0 + tile) * kTile, (int64_t)ks * kKBytes, sa);
    lb.issue(t0, (int64_t)ks * kKBytes, sb);
  };
  auto commit = [&](char* sa, char* sb) {
    if constexpr (!Q4) la.commit(sa);
    lb.commit(sb);
  };
  // ks == nk: the zero step of an odd nk (gemm_run_q4k); B then reads nothing (an empty range).
  auto issue_a = [&](auto set, int tile, int ks) {
    if constexpr (Q4)
      la.template issue<decltype(set)::value>((int64_t)(tile0 + tile) * kTile,
                                              (int64_t)min(ks, nk - 1) * E::kBK, ks < nk);
  };
  auto commit_a = [&](auto set, char* sa, auto w0, auto w1) {
    if constexpr (Q4)
      la.template commit_words<decltype(set)::value, decltype(w0)::value, decltype(w1)::value>(sa);
  };
  auto issue_b = [&](int, int ks, char* sb) {
    const bool live = ks < nk;
    lb.issue(live ? t0 : a.M, live ? (int64_t)ks * kKBytes : 0, sb);
  };
  auto epi = [&](int tile, f32x16(&acc)[4][2]) {
    const int64_t vt0 = (int64_t)(tile0 + tile) * kTile;
    const int64_t vw0 = vt0 + wm * 128;              // first vocabulary row of this wave
    const bool tail = vt0 + kTile > a.V;
    float rmax = kNegInf;
    // u = z * log2e (or (z - cap) * log2e under a softcap), masked past V on the last tile only.
    // The uniform branch on the tail encloses the whole epilogue, so that the per-element masks
    // exist on that path alone. Values are recomputed from the accumulators in each pass.
    auto run = [&](auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      // Valid rows of the wave, less this lane's row offset 4 (l / 32), so that each element's test
      // compares a compile-time constant (nothing per element is kept live across the K loop).
      const int lim = kMasked ? (int)min<int64_t>(max<int64_t>(a.V - vw0, 0), 128) - 4 * (l >> 5)
                              : 128;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        // Each pass over the elements tests against its own copy of the limit, opaque to the
        // compiler, so the tests sit where they are used instead of 64 lane masks shared between
        // passes staying live in scalar registers.
        auto fresh_lim = [&]() {
          int v = lim;
          if constexpr (kMasked) asm volatile("" : "+v"(v));
          return v;
        };
        auto keep_below = [](int lim_p, int mb, int r) {
          return !kMasked || mb * 32 + 8 * (r >> 2) + (r & 3) < lim_p;
        };
        float ref = m[nb];
        if (kRunMax) {
          const int lim_max = fresh_lim();
          float tmax = kNegInf;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (keep_below(lim_max, mb, r)) tmax = fmaxf(tmax, acc[mb][nb][r]);
          // z is monotone in raw: the tile's largest z * log2e (-cap log2e when no row is kept,
          // which adds no term and only moves the reference).
          const float zt = SOFTCAP ? __builtin_fmaf(sc.kz, sc.r_of(tmax), sc.cap * kLog2e) : tmax * kLog2e;
          const float mn = fmaxf(m[nb], zt);
          if (mn != kNegInf) {
            s[nb] *= exp2_(m[nb] - mn);   // m = -inf gives 0
            m[nb] = mn;
          }
          ref = m[nb];
        }
        float acc_s = 0.f;
        // u = z log2e - ref. Fixed reference: (z - cap) log2e = kz r. Running max under a softcap:
        // kz r + (cap log2e - ref).
        const float ub = SOFTCAP ? sc.cap * kLog2e - ref : -ref;
        if (ref != kNegInf) {
          const int lim_sum = fresh_lim();
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float raw = acc[mb][nb][r];
              const float x = !SOFTCAP ? __builtin_fmaf(raw, kLog2e, ub)
                              : (kRunMax ? __builtin_fmaf(sc.kz, sc.r_of(raw), ub) : sc.kz * sc.r_of(raw));
              const float e = exp2_(x);
              const bool keep = keep_below(lim_sum, mb, r);
              acc_s += keep ? e : 0.f;
              if constexpr (TMAX) rmax = fmaxf(rmax, keep ? raw : kNegInf);
            }
        }
        s[nb] += acc_s;
        // Target capture: the one lane holding (v = y, t) writes z[y] to logp[t].
        const int64_t off = (int64_t)y[nb] - vw0;
        const bool mine = off >= 0 && off < 128 && (((int)off >> 2) & 1) == (l >> 5);
        if (__builtin_expect(__ballot(mine) != 0, 0)) {
          if (mine) {
            const int o = (int)off, mb = o >> 5, ro = o & 31;
            const int r = ((ro >> 3) << 2) | (ro & 3);
            float zsel = 0.f;
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
#pragma unroll
              for (int rr = 0; rr < 16; ++rr)
                if (mm == mb && rr == r) zsel = acc[mm][nb][rr];
            const float z = SOFTCAP ? sc.cap - 2.f * sc.cap * sc.r_of(zsel) : zsel;
            a.logp[tok_of(nb)] = z;
          }
        }
      }
    };
    if (tail) run(std::true_type{});
    else run(std::false_type{});
    if constexpr (TMAX) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o));
      // In the 4-bit loop the wave index is made uniform (readfirstlane), so that no per-lane
      // 64-bit address is held across the K loop for this once-per-tile store.
      int wi = w;
      if constexpr (Q4) wi = __builtin_amdgcn_readfirstlane(w);
      if (l == 0) a.tmax[((int64_t)tb * a.n_vtiles + tile0 + tile) * 8 + wi] = rmax;
    }
  };
  constexpr bool kF8 = std::is_same<E, EFp8>::value;
  const int32_t sc_b = kF8 ? pack_row_exps<2>(a.h_exp, t0 + wn * 64, l & 31, a.M) : 0;   // fixed
  auto scales = [&, sc_b](int tile) {
    typename E::Scales sc{};
    if constexpr (kF8) {
      sc.a = pack_row_exps<4>(a.w_exp, (int64_t)(tile0 + tile) * kTile + wm * 128, l & 31, a.V);
      sc.b = sc_b;
    }
    return sc;
  };
  f32x16 acc[4][2];
  zero_acc(acc);
  if constexpr (Q4)
    gemm_run_q4k<true, Q4K2::kLoads>(smem, n_tiles, nk, issue_a, commit_a, issue_b, epi, acc);
  else gemm_run_scaled<E, true, true, true, true>(smem, n_tiles, nk, issue, commit, epi, scales, acc);

  // Combine the lane pair (l, l ^ 32), then the two m-waves, and write this split's partials.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float mo = __shfl_xor(m[nb], 32), so = __shfl_xor(s[nb], 32);
    if (kRunMax) {
      const float mn = fmaxf(m[nb], mo);
      if (mn != kNegInf) {
        s[nb] = s[nb] * exp2_(m[nb] - mn) + so * exp2_(mo - mn);
        m[nb] = mn;
      }
    } else {
      s[nb] += so;
    }
  }
  float2* red = (float2*)smem.a0;   // [256 tokens]
  if (wm == 1 && l < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) red[acc_n(wn, nb, l)] = make_float2(m[nb], s[nb]);
  }
  __syncthreads();
  if (wm == 0 && l < 32) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float2 o = red[acc_n(wn, nb, l)];
      float mm = m[nb], ss = s[nb];
      if (kRunMax) {
        const float mn = fmaxf(mm, o.x);
        if (mn != kNegInf) {
          ss = ss * exp2_(mm - mn) + o.y * exp2_(o.x - mn);
          mm = mn;
        }
      } else {
        ss += o.y;
      }
      const int64_t tok = tok_of(nb);
      if (tok < a.M) a.part[(int64_t)split * a.M + tok] = make_float2(mm, ss);
    }
  }
}

// Fills n floats with zeros (a kernel rather than hipMemsetAsync, so that a captured graph holds no
// memset node).
__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

// ------------------------------------------------------------------------------------------
// Merge the per-split partials: G = max_k m_k, S = sum_k s_k 2^(m_k - G), lse = (G + log2 S) ln 2.
// ------------------------------------------------------------------------------------------
// lse and logp of token t from the merged maximum G (log2 units) and sum S against it.
__device__ __forceinline__ void merge_finish(int64_t t, float G, float S, const int32_t* labels,
                                             int64_t V, int32_t ignore_index, float* logp,
                                             float* lse, uint32_t* status) {
  const float L = (G + log2_(S)) * kLn2;
  lse[t] = L;
  const int y = labels[t];
  if (y == ignore_index) {
    logp[t] = 0.f;
  } else if (y < 0 || (int64_t)y >= V) {
    logp[t] = 0.f;
    atomicOr(status, kStatusBadLabel);
  } else {
    logp[t] = logp[t] - L;
  }
}

// One thread per token, the splits in order: for few splits (large M).
__global__ __launch_bounds__(256) void merge_kernel(const float2* part, int nblk, int64_t M,
                                                    const int32_t* labels, int64_t V,
                                                    int32_t ignore_index, float* logp, float* lse,
                                                    uint32_t* status) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M) return;
  float G = kNegInf;
  for (int k = 0; k < nblk; ++k) G = fmaxf(G, part[(int64_t)k * M + t].x);
  float S = 0.f;
  for (int k = 0; k < nblk; ++k) {
    const float2 p = part[(int64_t)k * M + t];
    if (p.y > 0.f) S += p.y * exp2_(p.x - G);
  }
  merge_finish(t, G, S, labels, V, ignore_index, logp, lse, status);
}

// One wave per token, lane l taking splits l, l + 64, ...: for many splits (small M, where the
// forward spreads each token tile over up to 256 vocabulary splits and one thread per token would
// leave most of the chip idle behind long serial loops). The wave's maximum and sum are xor-shuffle
// butterflies, a fixed order.
__global__ __launch_bounds__(256) void merge_wide_kernel(const float2* part, int nblk, int64_t M,
                                                         const int32_t* labels, int64_t V,
                                                         int32_t ignore_index, float* logp,
                                                         float* lse, uint32_t* status) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // uniform per wave
  const int l = threadIdx.x & 63;
  if (t >= M) return;
  float G = kNegInf;
  for (int k = l; k < nblk; k += 64) G = fmaxf(G, part[(int64_t)k * M + t].x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) G = fmaxf(G, __shfl_xor(G, o));
  float S = 0.f;
  for (int k = l; k < nblk; k += 64) {
    const float2 p = part[(int64_t)k * M + t];
    if (p.y > 0.f) S += p.y * exp2_(p.x - G);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) S += __shfl_xor(S, o);
  if (l == 0) merge_finish(t, G, S, labels, V, ignore_index, logp, lse, status);
}

// ------------------------------------------------------------------------------------------
// Loss: one workgroup. Per-branch sums in f64 with fixed-order wave reductions, the scalar ORPO
// epilogue in f64 per pair, fixed-order sums over pairs, then g for every token.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ double log1mexp_d(double x, bool* clamped) {
  const double v = -expm1(x);
  if (!(v >= 1e-12)) {
    *clamped = true;
    return log(1e-12);
  }
  *clamped = false;
  return x > -0.6931471805599453 ? log(v) : log1p(-exp(x));
}

// Span offsets valid (0 <= off[0], off[i] <= off[i+1], off[n] <= M)? Checked by every thread of
// the workgroup on a strided share of the offsets. Thread 0 then resets the status word (or sets
// the bad-offsets bit), before a barrier, so that it precedes every later atomicOr into it.
__device__ __forceinline__ bool check_offsets(const int32_t* off, int n, int64_t M, uint32_t* status) {
  int b = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) b |= off[i + 1] < off[i];
  if (threadIdx.x == 0) b |= off[0] < 0 || (int64_t)off[n] > M;
  b = __syncthreads_or(b);
  if (threadIdx.x == 0) *status = b ? kStatusBadOffsets : 0u;
  __syncthreads();
  return b != 0;
}

// Sum of logp over the valid tokens of span s and their count, one wave per span (fixed order:
// each lane's tokens in order, then a fixed butterfly). Both loads are unconditional (in bounds)
// and the loop unrolled, so that several are in flight; an invalid token adds +0.0, which changes
// no sum.
__device__ __forceinline__ void span_sum(const int32_t* off, int s, const float* logp,
                                         const int32_t* labels, int32_t ignore, int64_t V,
                                         double* sum_out, long long* n_out) {
  const int l = threadIdx.x & 63;
  double sum = 0.0;
  long long n = 0;
  const int64_t end = off[s + 1];
#pragma unroll 4
  for (int64_t t = off[s] + l; t < end; t += 64) {
    const int y = labels[t];
    const float lp = logp[t];
    const bool ok = y != ignore && y >= 0 && (int64_t)y < V;
    sum += ok ? (double)lp : 0.0;
    n += ok ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o);
    n += __shfl_xor(n, o);
  }
  *sum_out = sum;
  *n_out = n;
}

// A fixed-order sum of n terms by one wave: lane l adds terms l, l + 64, ... in order, then a
// butterfly, after which every lane holds the same total (lanes l and l ^ o add the same two
// values at each level). Deterministic, and its loads are all in flight at once, unlike one
// thread's sequential loop.
template <class T, class F>
__device__ __forceinline__ T wave_sum(int n, F&& term) {
  const int l = threadIdx.x & 63;
  T s = T(0);
  for (int i = l; i < n; i += 64) s += term(i);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  return s;
}

// The per-token cotangent g[0, M), span by span in the waves' order of the sums (wave w takes
// spans w, w + 16, ...): per_span(s) gives span s's token function (its span constants read once),
// applied to each valid token of the span; invalid tokens and tokens outside every span get 0.
template <class PerSpan>
__device__ __forceinline__ void fill_g_by_span(const int32_t* off, int ns, int64_t M,
                                               const int32_t* labels, int32_t ignore, int64_t V,
                                               float* g, PerSpan&& per_span) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  for (int s = w; s < ns; s += 16) {
    auto tok = per_span(s);
    for (int64_t t = off[s] + l; t < off[s + 1]; t += 64) {
      const int y = labels[t];
      g[t] = y != ignore && y >= 0 && (int64_t)y < V ? tok(t) : 0.f;
    }
  }
  for (int64_t t = tid; t < off[0]; t += 1024) g[t] = 0.f;
  for (int64_t t = off[ns] + tid; t < M; t += 1024) g[t] = 0.f;
}

struct LossArgs {
  int64_t M, V;
  int32_t P;
  int32_t S;              // spans per pair: 2 = (chosen, rejected), 3 = (prompt, chosen, rejected)
  const int32_t* off;     // [S P + 1]
  const float* logp;
  const int32_t* labels;
  int32_t ignore_index;
  double lam;
  double* out;            // [5 + 2P] (S = 2) or [5 + 3P] (S = 3)
  float* g;               // [M]
  double* ell;            // ws [S P] span means
  double* sum;            // ws [S P] span sums
  double* dl;             // ws [S P] dL / d ell
  int64_t* cnt;           // ws [S P]
  double* pair;           // ws [3P]: log_odds, L_OR, accuracy bit
  uint32_t* status;
};

// Span means, the scalar ORPO epilogue and the per-token cotangent, in one workgroup. With S = 3 the
// NLL is the full-scope one: per pair, the token mean of -logp over the prompt span and the chosen
// response together, -(sum_q + sum_w) / (n_q + n_w), i.e. the combination -((P-1) pm + M lw) /
// ((P-1) + M) of the two span means (Training — design, §1 "The objective", sft_scope `full`); the
// odds ratio keeps the response means. A prompt span without a valid token is allowed (weight 0,
// reported mean 0); then every result equals the S = 2 one bit for bit.
__global__ __launch_bounds__(1024) void loss_kernel(LossArgs a) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int S = a.S, ns = S * a.P, nout = 5 + (S == 3 ? 3 : 2) * a.P;
  const double nan = __builtin_nan("");
  if (check_offsets(a.off, ns, a.M, a.status)) {
    for (int i = tid; i < nout; i += 1024) a.out[i] = nan;
    for (int64_t t = tid; t < a.M; t += 1024) a.g[t] = nan;
    return;
  }
  // Span sums: wave w takes spans w, w + 16, ...
  for (int b = w; b < ns; b += 16) {
    double sum;
    long long n;
    span_sum(a.off, b, a.logp, a.labels, a.ignore_index, a.V, &sum, &n);
    if (l == 0) {
      const bool prompt = S == 3 && b % 3 == 0;
      a.cnt[b] = n;
      a.sum[b] = sum;
      a.ell[b] = n > 0 ? sum / (double)n : (prompt ? 0.0 : nan);
      if (n == 0 && !prompt) atomicOr(a.status, kStatusEmptyBranch);
    }
  }
  __syncthreads();
  // Per pair: log-odds, L_OR, and dL/d ell for every span.
  for (int p = tid; p < a.P; p += 1024) {
    const int cw_i = S * p + S - 2, cr_i = S * p + S - 1;
    const double lw = a.ell[cw_i], lr = a.ell[cr_i];
    bool cw, cr;
    const double ow = log1mexp_d(lw, &cw), orr = log1mexp_d(lr, &cr);
    const double z = (lw - lr) - (ow - orr);
    const double lor = fmax(-z, 0.0) + log1p(exp(-fabs(z)));                 // softplus(-z)
    const double oms = z >= 0 ? exp(-z) / (1.0 + exp(-z)) : 1.0 / (1.0 + exp(z));   // 1 - sigmoid(z)
    const double fw = cw ? 1.0 : -1.0 / expm1(lw);
    const double fr = cr ? 1.0 : -1.0 / expm1(lr);
    if (S == 3) {
      const double tot = (double)(a.cnt[3 * p] + a.cnt[3 * p + 1]);
      a.dl[3 * p] = -((double)a.cnt[3 * p] / tot) / (double)a.P;
      a.dl[cw_i] = (-((double)a.cnt[cw_i] / tot) - a.lam * oms * fw) / (double)a.P;
      a.out[5 + 2 * a.P + p] = a.ell[3 * p];
    } else {
      a.dl[cw_i] = (-1.0 - a.lam * oms * fw) / (double)a.P;
    }
    a.dl[cr_i] = (a.lam * oms * fr) / (double)a.P;
    a.pair[p] = z;
    a.pair[a.P + p] = lor;
    a.pair[2 * a.P + p] = lw > lr ? 1.0 : 0.0;
    a.out[5 + p] = lw;
    a.out[5 + a.P + p] = lr;
  }
  __syncthreads();
  if (w == 0) {
    const double nll = -wave_sum<double>(a.P, [&](int p) {
      return S == 3 ? (a.sum[3 * p] + a.sum[3 * p + 1]) / (double)(a.cnt[3 * p] + a.cnt[3 * p + 1])
                    : a.ell[2 * p];
    });
    const double orv = wave_sum<double>(a.P, [&](int p) { return a.pair[a.P + p]; });
    const double acc = wave_sum<double>(a.P, [&](int p) { return a.pair[2 * a.P + p]; });
    const double mar = wave_sum<double>(a.P, [&](int p) { return a.pair[p]; });
    if (l == 0) {
      const double P = (double)a.P;
      a.out[0] = nll / P + a.lam * (orv / P);
      a.out[1] = nll / P;
      a.out[2] = orv / P;
      a.out[3] = acc / P;
      a.out[4] = mar / P;
    }
  }
  // g_t = (dL/d ell_s) / n_s for a valid token of span s.
  fill_g_by_span(a.off, ns, a.M, a.labels, a.ignore_index, a.V, a.g, [&](int s) {
    const float gs = a.cnt[s] > 0 ? (float)(a.dl[s] / (double)a.cnt[s]) : 0.f;
    return [gs](int64_t) { return gs; };
  });
}

// ------------------------------------------------------------------------------------------
// Backward. The work is a sequence of items (token chunk c0 of C_cur tokens) x (vocabulary block v0
// of BV_cur rows). Item i's coefficients go to coefficient buffer i % 2; launch i holds the
// coefficient tiles of item i together with the dh / dW tiles of item i - 1 (which read buffer
// (i - 1) % 2, written by the previous launch), longest tiles first, so the short coefficient tiles
// fill the tail of the long GEMM tiles. Every accumulation into dh and dW has a fixed order.
// ------------------------------------------------------------------------------------------
struct BwdItem {
  int64_t c0, C_cur;      // token chunk [c0, c0 + C_cur)
  int64_t v0, BV_cur;     // vocabulary block [v0, v0 + BV_cur)
  void* coeff;            // [C, BVb] of E::T, token-major
  uint8_t* fdh;           // coefficient filter flags for dh: [C/256][BVb/64][4] (null: filter off)
  uint8_t* fdw;           // ... and for dW: [BVb/256][C/64][2]
  int32_t n_tiles;        // workgroups of this item in the launch (coefficient: n_vt * n_tt; GEMM: dh + dW)
  int32_t n_vt, n_tt;     // 256-tiles along vocabulary and tokens
  int32_t n_dh;           // dh workgroups (GEMM item: dh tiles x dh_split); dW tiles are n_tiles - n_dh
  int32_t dh_split;       // K ranges per dh tile (1: none); each writes an fp32 partial to dh_part
  float* dh_part;         // [dh_split][C][d] partial sums over chunk rows (dh_split > 1)
  int64_t dh_part_pitch;  // elements from one split's partial to the next (C d)
  int32_t dh_first, dw_first;
  int32_t dh_last;        // the chunk's last vocabulary block (bf16 dh is written then)
};

struct BwdArgs {
  const void* h;
  const void* w;
  Q4Weight q4;
  const void* hq;         // FP8 logit operands (coefficient recompute of the FP8 head), else null
  const void* wq;
  const uint8_t* h_exp;
  const uint8_t* w_exp;
  const int32_t* labels;
  const float* lse;
  const float* g;
  float* dh;              // [M, d] fp32, or null when dh16 is set
  uint16_t* dh16;         // [M, d] bf16 output (ORPO_DH_BF16), else null
  float* dh_acc;          // [C, d] fp32 accumulator of the chunk for bf16 dh over several blocks
  float* dW;              // [V, d] or null
  int64_t M, d, V;
  int64_t BVb;            // row pitch of a coefficient buffer (elements)
  float cap;
  int32_t ignore_index;
  int32_t n_jt;           // 256-tiles along d
  float skip_eps;         // coefficient filter threshold (0: exact backward)
  int32_t nsl_v, nsl_t;   // 64-wide vocabulary / token slices per coefficient buffer row / column
  const float* tmax;      // the forward's per-tile, per-wave raw maxima [M/256][V/256][8] (or null)
  int32_t n_vtiles;       // 256-tiles along the whole vocabulary
  BwdItem gm;             // dh / dW tiles (n_tiles = 0: none)
  BwdItem cf;             // coefficient tiles (n_tiles = 0: none)
};

// Phase 1: recompute a 256 x 256 logit tile (m = vocabulary, n = token) and write its coefficients
// coeff = g (onehot - softmax) sech^2 (bf16 or fp32) to the item's coefficient buffer. EL is the
// logit operands' format: E, or EFp8 for the FP8 head (its forward's operands, so that the
// recomputed logits are the ones its lse was taken over).
template <class E, bool Q4, bool SOFTCAP, bool SKIP, class EL>
__device__ __forceinline__ void coeff_tile(const Smem& smem, const BwdArgs& a, const BwdItem& it,
                                           int bid) {
  constexpr bool kF8 = std::is_same<EL, EFp8>::value;
  static_assert(!(kF8 && Q4), "FP8 logit operands come from a bf16 head");
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 2, wn = w & 3;
  // Plain round-robin order: consecutive tiles step along the vocabulary, so an XCD's ~32
  // concurrent tiles form a ~(8 vocabulary x 4 token) group sharing 12 operand slices.
  const int vt = bid % it.n_vt, tt = bid / it.n_vt;
  const int64_t vbase = it.v0 + (int64_t)vt * kTile;  // global vocabulary row of tile row 0
  const int64_t tbase = it.c0 + (int64_t)tt * kTile;  // global token of tile column 0
  const int64_t t_end = min(a.M, it.c0 + it.C_cur);
  const int64_t row_bytes = a.d * EL::kSize;
  const Softcap sc(SOFTCAP ? a.cap : 1.f);

  if constexpr (SKIP) {
    // Cold tile (the forward's block maxima): every coefficient obeys |coeff_tv| <= |g_t| p_tv
    // <= |g_t| 2^((zmax - lse_t) log2 e) off the label (sech^2 <= 1), with zmax the softcapped
    // largest raw logit the forward saw in this tile. When that bound is below eps for every
    // token and no token's label falls in the tile, the filter would drop all of the tile's blocks:
    // write its flags as zero and skip the recompute (the coefficients are then never read).
    if (a.tmax) {
      __shared__ float cold_b[4];
      __shared__ int cold_y[4];
      const int64_t tile_idx = ((tbase >> 8) * a.n_vtiles + (vbase >> 8)) * 8;
      float rmax = kNegInf;
#pragma unroll
      for (int i = 0; i < 8; ++i) rmax = fmaxf(rmax, a.tmax[tile_idx + i]);
      const float zmax = SOFTCAP ? sc.cap - 2.f * sc.cap * sc.r_of(rmax) : rmax;
      float b = 0.f;
      bool ylab = false;
      if (tid < kTile) {
        const int64_t tk = tbase + tid;
        const int y = tk < t_end ? a.labels[tk] : a.ignore_index;
        const bool yv = tk < t_end && y != a.ignore_index && y >= 0 && (int64_t)y < a.V;
        const float gt = yv ? a.g[tk] : 0.f;
        if (gt != 0.f) {
          b = fabsf(gt) * exp2_((zmax - a.lse[tk]) * kLog2e);
          ylab = (int64_t)y >= vbase && (int64_t)y < vbase + kTile;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) b = fmaxf(b, __shfl_xor(b, o));
        const bool anyy = __ballot(ylab) != 0;
        if (l == 0) {
          cold_b[w] = b;
          cold_y[w] = anyy;
        }
      }
      __syncthreads();
      const float bound = fmaxf(fmaxf(cold_b[0], cold_b[1]), fmaxf(cold_b[2], cold_b[3]));
      const bool cold = !(cold_y[0] | cold_y[1] | cold_y[2] | cold_y[3]) &&
                        bound * 1.001f < a.skip_eps;      // margin for exp2's rounding
      if (cold) {
        if (l == 0) {
          uint8_t* fh = it.fdh + ((int64_t)tt * a.nsl_v + 4 * vt + 2 * wm) * 4 + wn;
          fh[0] = 0;
          fh[4] = 0;
          it.fdw[((int64_t)vt * a.nsl_t + 4 * tt + wn) * 2 + wm] = 0;
        }
        return;
      }
    }
  }

  typedef typename std::conditional<Q4, Q4K2, DmaKS<EL::kSwzShift, EL::kSwzK>>::type LoaderA;
  LoaderA la;
  DmaKS<EL::kSwzShift, EL::kSwzK> lb;
  if constexpr (Q4) la.init(a.q4); else la.init(kF8 ? a.wq : a.w, row_bytes, a.V);
  lb.init(kF8 ? a.hq : a.h, row_bytes, t_end);
  const int nk = (int)(a.d / EL::kBK);
  // As in the forward: 4-bit words through gemm_run_q4k's two register sets, the rest direct.
  auto issue = [&](int, int ks, char* sa, char* sb) {
    if constexpr (!Q4) la.issue(vbase, (int64_t)ks * kKBytes, sa);
    lb.issue(tbase, (int64_t)ks * kKBytes, sb);
  };
  auto issue_a = [&](auto set, int, int ks) {
    if constexpr (Q4)
      la.template issue<decltype(set)::value>(vbase, (int64_t)min(ks, nk - 1) * E::kBK, ks < nk);
  };
  auto commit_a = [&](auto set, char* sa, auto w0, auto w1) {
    if constexpr (Q4)
      la.template commit_words<decltype(set)::value, decltype(w0)::value, decltype(w1)::value>(sa);
  };
  auto issue_b = [&](int, int ks, char* sb) {
    const bool live = ks < nk;
    lb.issue(live ? tbase : t_end, live ? (int64_t)ks * kKBytes : 0, sb);
  };
  auto commit = [&](char* sa, char* sb) {
    if constexpr (!Q4) la.commit(sa);
    lb.commit(sb);
  };
  auto scales = [&](int) {
    typename EL::Scales s{};
    if constexpr (kF8) {
      s.a = pack_row_exps<4>(a.w_exp, vbase + wm * 128, l & 31, a.V);
      s.b = pack_row_exps<2>(a.h_exp, tbase + wn * 64, l & 31, t_end);
    }
    return s;
  };
  f32x16 acc[4][2];
  zero_acc(acc);
  auto nop = [](int, f32x16(&)[4][2]) {};
  if constexpr (Q4) gemm_run_q4k<false, Q4K2::kLoads>(smem, 1, nk, issue_a, commit_a, issue_b, nop, acc);
  else gemm_run_scaled<EL, true, true, false, true>(smem, 1, nk, issue, commit, nop, scales, acc);

  typedef typename E::T T;
  T* out = (T*)it.coeff;
  float cmax[2] = {0.f, 0.f};   // max |coeff| of this lane in vocabulary slices 2 wm and 2 wm + 1
  const int64_t vw0 = vbase + wm * 128;            // first vocabulary row of this wave
  // Valid rows of the wave less this lane's row offset 4 (l / 32), as in the forward, so that the
  // tail tile's mask compares compile-time constants.
  const int lim = (int)min<int64_t>(max<int64_t>(a.V - vw0, 0), 128) - 4 * (l >> 5);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = acc_n(wn, nb, l);
    const int64_t tk = tbase + n;
    const bool tv = tk < t_end;
    const int y = tv ? a.labels[tk] : a.ignore_index;
    const bool yv = tv && y != a.ignore_index && y >= 0 && (int64_t)y < a.V;   // else: ignored
    const float gt = yv ? a.g[tk] : 0.f;
    // An ignored token gets L2 = +inf: every exponential below is then exactly 0, whatever its
    // logits, so its coefficients are 0 (never 0 * inf = NaN from an overflowing exp2).
    const float L2 = yv ? a.lse[tk] * kLog2e : __builtin_huge_valf();
    // Off the label, coeff = -g p sech^2. Under a softcap, with rr = 1 / (1 + 2^(raw c1)) (so
    // tanh = 1 - 2 rr, z log2e = cap log2e + kz rr, sech^2 = 4 rr (1 - rr)), that is
    //   coeff = G (rr - rr^2) 2^(kz rr + B),   G = -4 g,  B = cap log2e - L2  (per token);
    // without one, coeff = G 2^(raw log2e + B) with G = -g, B = -L2. The exponent is
    // (z - lse) log2e <= 0 as one sum, so no intermediate factor leaves float range, for any
    // softcap. The label's own entry adds g sech^2 (patched below).
    const float G = SOFTCAP ? -4.f * gt : -gt;
    const float B = SOFTCAP ? sc.cap * kLog2e - L2 : -L2;
    T* row = out + (tk - it.c0) * a.BVb + (vbase - it.v0);
    auto body = [&](auto masked_tag) {
      constexpr bool kMasked = decltype(masked_tag)::value;
      // This half's own copy of the limit, opaque to the compiler, so that each element is tested
      // where it is stored rather than through 64 lane masks kept live in scalar registers.
      int lim_nb = lim;
      if constexpr (kMasked) asm volatile("" : "+v"(lim_nb));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          float vals[4];
#pragma unroll
          for (int ri = 0; ri < 4; ++ri) {
            const int r = rg * 4 + ri;
            const float raw = acc[mb][nb][r];
            float c;
            if (SOFTCAP) {
              const float rr = sc.r_of(raw);
              c = G * (__builtin_fmaf(-rr, rr, rr) * exp2_(__builtin_fmaf(sc.kz, rr, B)));
            } else {
              c = G * exp2_(__builtin_fmaf(raw, kLog2e, B));
            }
            if (kMasked && !(mb * 32 + 8 * rg + ri < lim_nb)) c = 0.f;
            vals[ri] = c;
            if constexpr (SKIP) cmax[mb >> 1] = fmaxf(cmax[mb >> 1], fabsf(c));
          }
          // 4 consecutive vocabulary entries of token tk.
          const int m0 = acc_m(wm, mb, rg * 4, l);
          if constexpr (sizeof(T) == 2) {
            u32x2 pk;
            pk[0] = pack_bf16x2(vals[0], vals[1]);
            pk[1] = pack_bf16x2(vals[2], vals[3]);
            *(u32x2*)(row + m0) = pk;
          } else {
            *(f32x4*)(row + m0) = f32x4{vals[0], vals[1], vals[2], vals[3]};
          }
        }
    };
    if (vbase + kTile > a.V) body(std::true_type{}); else body(std::false_type{});
    // The label's entry: the one lane holding (v = y, t) rewrites it as g (1 - p) sech^2, after its
    // earlier store to the same address has completed.
    const int64_t off = (int64_t)y - vw0;
    const bool mine = yv && off >= 0 && off < 128 && (((int)off >> 2) & 1) == (l >> 5);
    if (__builtin_expect(__ballot(mine) != 0, 0)) {
      if (mine) {
        const int o = (int)off, mbl = o >> 5, ro = o & 31;
        const int rl = ((ro >> 3) << 2) | (ro & 3);
        float raw = 0.f;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
#pragma unroll
          for (int rr_ = 0; rr_ < 16; ++rr_)
            if (mm == mbl && rr_ == rl) raw = acc[mm][nb][rr_];
        float zl2, slope;
        if (SOFTCAP) {
          const float rr = sc.r_of(raw);
          zl2 = (sc.cap - 2.f * sc.cap * rr) * kLog2e;
          slope = 4.f * rr * (1.f - rr);
        } else {
          zl2 = raw * kLog2e;
          slope = 1.f;
        }
        const float c = gt * (1.f - exp2_(zl2 - L2)) * slope;
        if constexpr (SKIP) cmax[mbl >> 1] = fmaxf(cmax[mbl >> 1], fabsf(c));
        vm_wait();
        if constexpr (sizeof(T) == 2) {
          *(uint16_t*)(row + (vw0 - vbase) + o) = (uint16_t)(pack_bf16x2(c, 0.f) & 0xffffu);
        } else {
          row[(vw0 - vbase) + o] = c;
        }
      }
    }
  }
  // Coefficient filter: this wave covers 64 tokens (slice wn of the tile) x 128 vocabulary entries
  // (slices 2 wm, 2 wm + 1); one flag byte per (token block, vocabulary slice, wave) for dh and per
  // (vocabulary block, token slice, wave) for dW, so every byte has exactly one writer.
  if constexpr (SKIP) {
    const bool f0 = __ballot(cmax[0] >= a.skip_eps) != 0, f1 = __ballot(cmax[1] >= a.skip_eps) != 0;
    if (l == 0) {
      uint8_t* fh = it.fdh + ((int64_t)tt * a.nsl_v + 4 * vt + 2 * wm) * 4 + wn;
      fh[0] = f0;
      fh[4] = f1;
      it.fdw[((int64_t)vt * a.nsl_t + 4 * tt + wn) * 2 + wm] = f0 || f1;
    }
  }
}

// With the coefficient filter on: the K steps (64-wide slices) whose flag bytes are not all zero,
// compacted in order into `list`; returns their count. Step s's flags are flags[s * parts + q].
__device__ __forceinline__ int build_klist(const uint8_t* flags, int nk, int parts, uint16_t* list,
                                           int* wave_tot) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  int total = 0;
  for (int base = 0; base < nk; base += kThreads) {
    const int s = base + tid;
    bool f = false;
    if (s < nk)
      for (int q = 0; q < parts; ++q) f |= flags[(int64_t)s * parts + q] != 0;
    const uint64_t m = __ballot(f);
    if (l == 0) wave_tot[w] = __popcll(m);
    __syncthreads();
    int off = total;
    for (int i = 0; i < w; ++i) off += wave_tot[i];
    int add = 0;
    for (int i = 0; i < kThreads / 64; ++i) add += wave_tot[i];
    if (f) list[off + __popcll(m & ((1ull << l) - 1ull))] = (uint16_t)s;
    total += add;
    __syncthreads();
  }
  return total;
}

// The first position of the ascending run list [0, n) whose step is >= v (n if none).
__device__ __forceinline__ int klist_lower_bound(const uint16_t* list, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int)list[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Row offset of accumulator element r within its 32 x 32 block (acc_m(wm, mb, r, l) - acc_m(wm, mb, 0, l)).
__device__ __forceinline__ int acc_dr(int r) { return 8 * (r >> 2) + (r & 3); }

// dh / dW tile store: out (+)= acc in fp32 (first: overwrite). A whole tile (the usual case) goes
// through a buffer descriptor over its 256 rows: each 32 x 32 block is one per-lane offset plus a
// uniform row offset per element, and its 16 previous values are all read before any is added, so
// a lane waits for memory 8 times per tile. Element by element (the tail path) each read is its
// own round trip.
template <class E>
__device__ __forceinline__ void store_out(float* out, int64_t ld, int64_t row0, int64_t n_rows,
                                          int64_t col0, int64_t n_cols, bool first,
                                          const f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 2, wn = w & 3;
  if (row0 + kTile <= n_rows && col0 + kTile <= n_cols) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc((const char*)(out + row0 * ld + col0), (int64_t)kTile * ld * 4);
    const int ldb = (int)(ld * 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int vo = acc_m(wm, mb, 0, l) * ldb + acc_n(wn, nb, l) * 4;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[mb][nb][r];
        if (!first) {
          float prev[16];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            prev[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo, acc_dr(r) * ldb, 0));
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = prev[r] + v[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[r]), rs, vo, acc_dr(r) * ldb, 0);
      }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t col = col0 + acc_n(wn, nb, l);
    if (col >= n_cols) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + acc_m(wm, mb, r, l);
        if (row < n_rows) {
          float* p = out + row * ld + col;
          *p = first ? acc[mb][nb][r] : *p + acc[mb][nb][r];
        }
      }
  }
}

// bf16 output of an fp32 tile: out16 = bf16(acc + prev) (prev: the chunk's fp32 accumulator rows,
// or nothing on the first block), rounded to nearest even once.
__device__ __forceinline__ void store_out_bf16(uint16_t* out16, const float* prev, int64_t ld,
                                               int64_t row0, int64_t prow0, int64_t n_rows,
                                               int64_t col0, int64_t n_cols,
                                               const f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 2, wn = w & 3;
  if (row0 + kTile <= n_rows && col0 + kTile <= n_cols) {   // whole tile: as store_out
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(prev ? (const char*)(prev + prow0 * ld + col0) : nullptr, prev ? (int64_t)kTile * ld * 4 : 0);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc((const char*)(out16 + row0 * ld + col0), (int64_t)kTile * ld * 2);
    const int ldb = (int)(ld * 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int m0 = acc_m(wm, mb, 0, l), n = acc_n(wn, nb, l);
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = acc[mb][nb][r];
        if (prev) {
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            pv[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, m0 * ldb + n * 4,
                                                                                  acc_dr(r) * ldb, 0));
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = pv[r] + v[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16x2(v[r], 0.f) & 0xffffu), ro,
                                                m0 * (ldb / 2) + n * 2, acc_dr(r) * (ldb / 2), 0);
      }
    return;
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t col = col0 + acc_n(wn, nb, l);
    if (col >= n_cols) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = acc_m(wm, mb, r, l);
        if (row0 + m < n_rows) {
          const float v = prev ? prev[(prow0 + m) * ld + col] + acc[mb][nb][r] : acc[mb][nb][r];
          out16[(row0 + m) * ld + col] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
        }
      }
  }
}

// Phase 2a: dh[c0 + i][j] (+)= sum_v coeff[i][v] W[v0 + v][j]   (m = token, n = hidden, k = vocabulary)
// With it.dh_split = S > 1 (few dh tiles, each with a long K), workgroup u of the dh range runs
// split s = u / n_tiles of tile u % n_tiles: the K steps [nk s / S, nk (s + 1) / S) (under the
// coefficient filter, those of its run list), and stores its fp32 sum as partial s;
// dh_reduce_kernel then adds the S partials in split order. The ranges are of step indices, not
// of run positions, so a filter that drops only all-zero steps sums the same steps per split as
// the exact backward and gives the same bits.
template <class E, bool Q4, bool SKIP>
__device__ __forceinline__ void dh_tile(const Smem& smem, const BwdArgs& a, const BwdItem& it, int bid,
                                        uint16_t* klist, int* wave_tot) {
  const int tid = threadIdx.x;
  const int64_t row_bytes = a.d * E::kSize;
  const int64_t cpitch = a.BVb * E::kSize;
  const int64_t t_end = min(a.M, it.c0 + it.C_cur);
  const int S = it.dh_split;
  const int u = xcd_remap(bid, it.n_dh);
  const int n_dh_tiles = it.n_dh / S;
  const int t = u % n_dh_tiles, split = u / n_dh_tiles;
  const int ti = t / a.n_jt, jt = t % a.n_jt;
  const int64_t i0 = (int64_t)ti * kTile, j0 = (int64_t)jt * kTile;
  const int64_t kv = ((it.BV_cur + kTile - 1) / kTile) * kTile;   // coefficient columns written
  const int nk = (int)((kv + E::kBK - 1) / E::kBK);
  const int64_t v_end = min(a.V, it.v0 + it.BV_cur);
  DmaK la;                                                          // coeff [i][v], K-major
  la.init(it.coeff, cpitch, it.C_cur);
  typedef typename std::conditional<Q4, Q4N2, DmaMN<E>>::type LoaderB;
  LoaderB lb;                                                       // W [v][j], N-major
  if constexpr (Q4) lb.init(a.q4, v_end);
  else lb.init((const char*)a.w + it.v0 * row_bytes, row_bytes, v_end - it.v0);   // block rows
  // Coefficient filter: run only the vocabulary slices some coefficient of this token tile needs.
  constexpr bool filt = SKIP;
  const int n_all = filt ? build_klist(it.fdh + (int64_t)ti * a.nsl_v * 4, nk, 4, klist, wave_tot) : nk;
  // This workgroup's run positions [kb, kb + n_run): its K steps' range, located in the ascending
  // run list under the filter.
  const int lo = (int)((int64_t)nk * split / S), hi = (int)((int64_t)nk * (split + 1) / S);
  const int kb = filt ? __builtin_amdgcn_readfirstlane(klist_lower_bound(klist, n_all, lo)) : lo;
  const int n_run = (filt ? __builtin_amdgcn_readfirstlane(klist_lower_bound(klist, n_all, hi)) : hi) - kb;
  // The vocabulary step of run position kb + ks (positions past n_run: the last one, in bounds).
  auto step_of = [&](int ks) {
    const int pos = kb + min(ks, n_run - 1);
    return filt ? __builtin_amdgcn_readfirstlane(klist[pos]) : pos;
  };
  f32x16 acc[4][2];
  zero_acc(acc);
  if constexpr (Q4) {
    // gemm_run_q4n: positions ks >= n_run (its zero step and the loads past the end) stage zeros.
    auto issue_a = [&](int ks, char* sa) {
      const bool live = ks < n_run;
      la.issue(live ? i0 : it.C_cur, live ? (int64_t)step_of(ks) * E::kBK * E::kSize : 0, sa);
    };
    auto issue_b = [&](auto set, int ks) {
      lb.template issue<decltype(set)::value>(it.v0 + (int64_t)step_of(ks) * E::kBK, j0, ks < n_run);
    };
    auto commit_b = [&](auto set, char* sb, auto w0, auto w1) {
      lb.template commit_words<decltype(set)::value, decltype(w0)::value, decltype(w1)::value>(sb);
    };
    gemm_run_q4n<Q4N2::kLoads>(smem, n_run, issue_a, issue_b, commit_b, acc);
  } else {
    auto issue = [&](int, int ks, char* sa, char* sb) {
      const int pos = kb + ks;
      const int64_t k0 = (int64_t)(filt ? __builtin_amdgcn_readfirstlane(klist[pos]) : pos) * E::kBK;
      la.issue(i0, k0 * E::kSize, sa);
      lb.issue(k0, j0 * E::kSize, sb);
    };
    auto commit = [&](char* sa, char* sb) {
      la.commit(sa);
      lb.commit(sb);
    };
    auto nop = [](int, f32x16(&)[4][2]) {};
    gemm_run<E, true, false, false, !SKIP>(smem, 1, n_run, issue, commit, nop, acc);
  }
  (void)tid;
  if (S > 1) {   // every split stores its partial (the reduction reads all of them), zeros included
    store_out<E>(it.dh_part + split * it.dh_part_pitch, a.d, i0, t_end - it.c0, j0, a.d, true, acc);
    return;
  }
  if (!a.dh16) {
    if (n_run > 0 || it.dh_first)
      store_out<E>(a.dh, a.d, it.c0 + i0, t_end, j0, a.d, it.dh_first != 0, acc);
  } else if (it.dh_last) {   // bf16 dh: sum in fp32 over the chunk's blocks, round once at the end
    store_out_bf16(a.dh16, it.dh_first ? nullptr : a.dh_acc, a.d, it.c0 + i0, i0, t_end, j0, a.d,
                   acc);
  } else if (n_run > 0 || it.dh_first) {
    store_out<E>(a.dh_acc, a.d, i0, t_end - it.c0, j0, a.d, it.dh_first != 0, acc);
  }
}

// The split dh tiles' partials of the chunk's rows, added in split order, then stored as an
// unsplit tile stores its sum: dh overwritten on the chunk's first vocabulary block and added to
// after it; bf16 dh through the chunk's fp32 accumulator, rounded once on the last block.
__global__ __launch_bounds__(256) void dh_reduce_kernel(BwdArgs a) {
  const BwdItem& it = a.gm;
  const int64_t n = (min(a.M, it.c0 + it.C_cur) - it.c0) * a.d;
  const int S = it.dh_split;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    float v = it.dh_part[e];
    for (int s = 1; s < S; ++s) v += it.dh_part[s * it.dh_part_pitch + e];
    if (!a.dh16) {
      float* p = a.dh + it.c0 * a.d + e;
      *p = it.dh_first ? v : *p + v;
    } else if (it.dh_last) {
      const float w = it.dh_first ? v : a.dh_acc[e] + v;
      a.dh16[it.c0 * a.d + e] = (uint16_t)(pack_bf16x2(w, 0.f) & 0xffffu);
    } else {
      a.dh_acc[e] = it.dh_first ? v : a.dh_acc[e] + v;
    }
  }
}

// Phase 2b: dW[v0 + v][j] (+)= sum_i coeff[i][v] h[c0 + i][j]   (m = vocabulary, n = hidden, k = token)
template <class E, bool SKIP>
__device__ __forceinline__ void dw_tile(const Smem& smem, const BwdArgs& a, const BwdItem& it, int bid,
                                        uint16_t* klist, int* wave_tot) {
  const int64_t row_bytes = a.d * E::kSize;
  const int64_t cpitch = a.BVb * E::kSize;
  const int64_t t_end = min(a.M, it.c0 + it.C_cur);
  const int t = xcd_remap(bid, it.n_tiles - it.n_dh);
  const int vt = t / a.n_jt, jt = t % a.n_jt;
  const int64_t vl0 = (int64_t)vt * kTile, j0 = (int64_t)jt * kTile;
  const int nk = (int)((it.C_cur + E::kBK - 1) / E::kBK);
  DmaMN<E> la;                                                      // coeff [i][v], M-major
  la.init(it.coeff, cpitch, it.C_cur);
  DmaMN<E> lb;                                                      // h [t][j], N-major
  lb.init((const char*)a.h + it.c0 * row_bytes, row_bytes, t_end - it.c0);   // chunk rows
  // Coefficient filter: run only the token slices some coefficient of this vocabulary tile needs.
  constexpr bool filt = SKIP;
  const int n_run = filt ? build_klist(it.fdw + (int64_t)vt * a.nsl_t * 2, nk, 2, klist, wave_tot) : nk;
  auto issue = [&](int, int ks, char* sa, char* sb) {
    const int step = filt ? __builtin_amdgcn_readfirstlane(klist[ks]) : ks;
    const int64_t k0 = (int64_t)step * E::kBK;
    la.issue(k0, vl0 * E::kSize, sa);
    lb.issue(k0, j0 * E::kSize, sb);
  };
  auto commit = [&](char* sa, char* sb) {
    la.commit(sa);
    lb.commit(sb);
  };
  f32x16 acc[4][2];
  zero_acc(acc);
  auto nop = [](int, f32x16(&)[4][2]) {};
  gemm_run<E, false, false, false, !SKIP>(smem, 1, n_run, issue, commit, nop, acc);
  if (n_run > 0 || it.dw_first)
    store_out<E>(a.dW, a.d, it.v0 + vl0, min(a.V, it.v0 + it.BV_cur), j0, a.d, it.dw_first != 0, acc);
}

// One launch of the backward pipeline: [dh tiles of gm | dW tiles of gm | coefficient tiles of cf].
// SKIP: the variant with the coefficient filter (orpo_head_desc.skip_eps > 0); the exact backward
// compiles without any of its code. F8: the coefficient tiles recompute the logits from the FP8
// operands (the dh / dW tiles are unchanged).
template <class E, bool Q4, bool SOFTCAP, bool SKIP, bool F8 = false>
__global__ __launch_bounds__(kThreads) void bwd_kernel(BwdArgs a) {
  ORPO_DECLARE_SMEM(smem);
  __shared__ uint16_t klist[SKIP ? kMaxKSteps : 1];   // K steps to run under the coefficient filter
  __shared__ int wave_tot[kThreads / 64];
  int b = blockIdx.x;
  if (b < a.gm.n_dh) {
    dh_tile<E, Q4, SKIP>(smem, a, a.gm, b, klist, wave_tot);
    return;
  }
  b -= a.gm.n_dh;
  if (b < a.gm.n_tiles - a.gm.n_dh) {
    if constexpr (!Q4) dw_tile<E, SKIP>(smem, a, a.gm, b, klist, wave_tot);
    return;
  }
  b -= a.gm.n_tiles - a.gm.n_dh;
  coeff_tile<E, Q4, SOFTCAP, SKIP, typename std::conditional<F8, EFp8, E>::type>(smem, a, a.cf, b);
}

}  // namespace orpo
