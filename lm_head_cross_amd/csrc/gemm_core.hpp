// gemm_core.hpp — the CDNA4 (gfx950) MFMA tile engine shared by every head kernel.
//
// One workgroup of 512 threads (8 wave64s) computes a 256 x 256 fp32 tile C[m][n] = sum_k
// A[m][k] B[k][n] with the 32x32 MFMA (bf16: v_mfma_f32_32x32x16_bf16, fp32: 4x
// v_mfma_f32_32x32x2f32 per 8-wide k group). Waves sit in a 2 (m) x 4 (n) grid; each owns a
// 128 x 64 sub-tile = 4 x 2 MFMA blocks = 128 accumulator registers per lane.
//
// Operands are staged through LDS in two stages of 128 bytes of K per row (64 bf16 / 32 fp32),
// double-buffered with one barrier per K step. Each operand tile keeps its global orientation:
//   K-major  ([rows][k], k contiguous)  -> LDS [256 rows][144 B], fragments via ds_read_b128;
//   MN-major ([k][cols], cols contiguous) -> LDS [BK rows][cols + pad], fragments via the gfx950
//            transposing LDS read (ds_read_b64_tr_b16) for bf16, 4 scalar reads for fp32.
// So the forward (A = W, B = h, both K-major), the dh GEMM (A = coeff K-major, B = W N-major) and
// the dW GEMM (A = coeff M-major, B = h N-major) all run on the same engine without any
// transposed copy in HBM. Row pitches are padded so that both the 16-byte fragment reads and the
// transposing reads hit distinct LDS banks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orpo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kTile = 256;              // tile extent in m and n
constexpr int kKBytes = 128;            // bytes of K per stage per row
constexpr int kKPitch = 144;            // K-major LDS row pitch (128 + 16 pad)
constexpr int kStageBytes = 36864;      // LDS bytes of one operand stage
constexpr int kLdsBytes = 4 * kStageBytes;
constexpr int kKGroups = 4;             // MFMA k groups per stage (bf16: 4 x 16, fp32: 4 x 8)

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ------------------------------------------------------------------------------------------
// Element policies: storage type, K per stage, MN-major pitch, fragment reads and the MFMA step.
// A fragment is 16 bytes per lane: for the 32-row block starting at row0, lane l holds row
// row0 + l % 32 and k slots kg*KG + (l / 32) * KG/2 + [0, KG/2) with KG = 16 (bf16) or 8 (fp32).
// Any consistent k-slot assignment gives the same sum, as long as A and B use the same one.
// ------------------------------------------------------------------------------------------
struct EBf16 {
  typedef __bf16 T;
  typedef bf16x8 Frag;
  static constexpr int kSize = 2;
  static constexpr int kBK = 64;        // K elements per stage
  static constexpr int kMnPitch = 576;  // MN-major LDS row pitch: 256 * 2 + 64 pad

  static __device__ __forceinline__ Frag frag_k(const char* s, int row0, int kg, int l) {
    return *(const Frag*)(s + (row0 + (l & 31)) * kKPitch + kg * 32 + (l >> 5) * 16);
  }
  // Transposing read: within each 16-lane group, source lane s reads 4 contiguous columns of row
  // (k0 + s/4); the hardware hands output lane j, slot i the element j%4 of source lane 4i + j/4,
  // i.e. column j of row k0 + i. Two reads give the 8 k slots of the lane's column.
  static __device__ __forceinline__ Frag frag_mn(const char* s, int col0, int kg, int l) {
    const int g = l >> 4, q = l & 15;
    const int row = kg * 16 + 8 * (g >> 1) + (q >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (q & 3);
    const char* p = s + row * kMnPitch + col * 2;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * kMnPitch));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(Frag, v);
  }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct EF32 {
  typedef float T;
  typedef f32x4 Frag;
  static constexpr int kSize = 4;
  static constexpr int kBK = 32;
  static constexpr int kMnPitch = 1056;  // 256 * 4 + 32 pad

  static __device__ __forceinline__ Frag frag_k(const char* s, int row0, int kg, int l) {
    return *(const Frag*)(s + (row0 + (l & 31)) * kKPitch + kg * 32 + (l >> 5) * 16);
  }
  static __device__ __forceinline__ Frag frag_mn(const char* s, int col0, int kg, int l) {
    const char* p = s + (kg * 8 + (l >> 5) * 4) * kMnPitch + (col0 + (l & 31)) * 4;
    Frag f;
    f[0] = *(const float*)(p);
    f[1] = *(const float*)(p + kMnPitch);
    f[2] = *(const float*)(p + 2 * kMnPitch);
    f[3] = *(const float*)(p + 3 * kMnPitch);
    return f;
  }
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------------------------------
// Global -> register -> LDS loaders. A tile is 2048 chunks of 16 bytes: 4 per thread.
// ------------------------------------------------------------------------------------------

// Dense tile of TR rows x (CPR * 16) bytes of a row-major global matrix; rows >= n_rows and
// bytes >= row_bytes are zero-filled (row_bytes is a multiple of 16).
template <int TR, int CPR>
struct DenseTile {
  static constexpr int kPer = TR * CPR / kThreads;
  static_assert(kPer * kThreads == TR * CPR, "tile must split evenly over the workgroup");
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const char* base, int64_t ld_bytes, int64_t row0,
                                       int64_t col0_bytes, int64_t n_rows, int64_t row_bytes,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / CPR, cc = c % CPR;
      const int64_t gr = row0 + r;
      const int64_t gb = col0_bytes + cc * 16;
      const bool ok = gr < n_rows && gb < row_bytes;
      const u32x4 x = *(const u32x4*)(base + (ok ? gr * ld_bytes + gb : 0));
      v[i] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* s, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kThreads;
      *(u32x4*)(s + (c / CPR) * pitch + (c % CPR) * 16) = v[i];
    }
  }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;   // round to nearest even
  return (uint32_t)__builtin_bit_cast(unsigned short, a) |
         ((uint32_t)__builtin_bit_cast(unsigned short, b) << 16);
}

// 8 codes of one packed word -> 8 bf16 (16 bytes): w = scale * q + bias in fp32, then RNE.
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, float scale, float bias) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = (float)((w >> (8 * i)) & 0xFu);
    const float q1 = (float)((w >> (8 * i + 4)) & 0xFu);
    o[i] = pack_bf16x2(__builtin_fmaf(scale, q0, bias), __builtin_fmaf(scale, q1, bias));
  }
  return o;
}

struct Q4Weight {
  const uint32_t* wq;        // [V, d/8]
  const uint16_t* scales;    // [V, d/64] bf16 bits
  const uint16_t* biases;
  int64_t V, d;
};

// 4-bit weights as a K-major operand: 256 vocabulary rows x 64 codes (one group) per stage.
// Thread tid owns row tid/2, codes [32*(tid%2), +32) of the stage's 64.
struct Q4KTile {
  u32x4 q;
  float scale, bias;
  __device__ __forceinline__ void load(const Q4Weight& W, int64_t row0, int64_t k0, int tid) {
    const int64_t gr = row0 + (tid >> 1);
    const bool ok = gr < W.V;
    const int64_t r = ok ? gr : 0;
    const u32x4 x = *(const u32x4*)(W.wq + r * (W.d >> 3) + (k0 >> 3) + (tid & 1) * 4);
    const int64_t gi = r * (W.d >> 6) + (k0 >> 6);
    const float s = bf16_bits_to_f32(W.scales[gi]), b = bf16_bits_to_f32(W.biases[gi]);
    q = ok ? x : u32x4{0u, 0u, 0u, 0u};
    scale = ok ? s : 0.f;
    bias = ok ? b : 0.f;
  }
  __device__ __forceinline__ void store(char* s, int /*pitch*/, int tid) const {
    char* p = s + (tid >> 1) * kKPitch + (tid & 1) * 64;
#pragma unroll
    for (int w = 0; w < 4; ++w) *(u32x4*)(p + w * 16) = dequant_word(q[w], scale, bias);
  }
};

// 4-bit weights as an N-major operand (rows = vocabulary = k, columns = hidden = n): 64 rows x
// 256 codes per stage. Thread tid owns row tid/8, codes [32*(tid%8), +32) of the tile's 256.
struct Q4NTile {
  u32x4 q;
  float scale, bias;
  __device__ __forceinline__ void load(const Q4Weight& W, int64_t k0, int64_t n0, int tid) {
    const int64_t gr = k0 + (tid >> 3);
    const int64_t gc = n0 + (tid & 7) * 32;
    const bool ok = gr < W.V && gc < W.d;
    const int64_t r = ok ? gr : 0, c = ok ? gc : 0;
    const u32x4 x = *(const u32x4*)(W.wq + r * (W.d >> 3) + (c >> 3));
    const int64_t gi = r * (W.d >> 6) + (c >> 6);
    const float s = bf16_bits_to_f32(W.scales[gi]), b = bf16_bits_to_f32(W.biases[gi]);
    q = ok ? x : u32x4{0u, 0u, 0u, 0u};
    scale = ok ? s : 0.f;
    bias = ok ? b : 0.f;
  }
  __device__ __forceinline__ void store(char* s, int pitch, int tid) const {
    char* p = s + (tid >> 3) * pitch + (tid & 7) * 64;
#pragma unroll
    for (int w = 0; w < 4; ++w) *(u32x4*)(p + w * 16) = dequant_word(q[w], scale, bias);
  }
};

// ------------------------------------------------------------------------------------------
// Compute one LDS stage into the wave's 4 x 2 accumulator blocks.
// ------------------------------------------------------------------------------------------
template <class E, bool AK, bool BK>
__device__ __forceinline__ void compute_stage(const char* sa, const char* sb, f32x16 (&acc)[4][2],
                                              int wm, int wn, int l) {
#pragma unroll
  for (int kg = 0; kg < kKGroups; ++kg) {
    typename E::Frag a[4], b[2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      a[mb] = AK ? E::frag_k(sa, wm * 128 + mb * 32, kg, l) : E::frag_mn(sa, wm * 128 + mb * 32, kg, l);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      b[nb] = BK ? E::frag_k(sb, wn * 64 + nb * 32, kg, l) : E::frag_mn(sb, wn * 64 + nb * 32, kg, l);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) E::mma(acc[mb][nb], a[mb], b[nb]);
  }
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
}

// The main loop over n_tiles consecutive output tiles of nk K steps each. `issue(tile, ks)`
// loads the global tiles of step (tile, ks) into the loaders' registers; `epi(tile, acc)` runs
// after the tile's last K step (before the loop's barrier; it must not touch LDS), then the
// accumulators are cleared unless kClear is false (single-tile callers read acc afterwards). The next step's global loads are in flight during each step's MFMAs.
template <class E, bool AK, bool BK, bool kClear = true, class LA, class LB, class Issue, class Epi>
__device__ __forceinline__ void gemm_run(char* smem, LA& la, LB& lb, int pa, int pb, int n_tiles,
                                         int nk, Issue&& issue, Epi&& epi, f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  char* sA0 = smem;
  char* sA1 = smem + kStageBytes;
  char* sB0 = smem + 2 * kStageBytes;
  char* sB1 = smem + 3 * kStageBytes;
  const int total = n_tiles * nk;
  if (total <= 0) return;
  issue(0, 0);
  la.store(sA0, pa, tid);
  lb.store(sB0, pb, tid);
  __syncthreads();
  int tile = 0, ks = 0;
  for (int it = 0; it < total; ++it) {
    const bool odd = it & 1;
    int nks = ks + 1, ntile = tile;
    if (nks == nk) { nks = 0; ++ntile; }
    const bool more = it + 1 < total;
    if (more) issue(ntile, nks);
    compute_stage<E, AK, BK>(odd ? sA1 : sA0, odd ? sB1 : sB0, acc, wm, wn, l);
    if (more) {
      la.store(odd ? sA0 : sA1, pa, tid);
      lb.store(odd ? sB0 : sB1, pb, tid);
    }
    if (nks == 0) {
      epi(tile, acc);
      if (kClear) zero_acc(acc);
    }
    __syncthreads();
    tile = ntile;
    ks = nks;
  }
}

// Position of accumulator element r of block (mb, nb) in the 256 x 256 tile.
__device__ __forceinline__ int acc_m(int wm, int mb, int r, int l) {
  return wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_n(int wn, int nb, int l) { return wn * 64 + nb * 32 + (l & 31); }

}  // namespace orpo
