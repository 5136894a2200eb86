// gemm_core.hpp — the CDNA4 (gfx950) MFMA tile engine shared by every head kernel.
//
// One workgroup of 512 threads (8 wave64s) computes a 256 x 256 fp32 tile C[m][n] = sum_k
// A[m][k] B[k][n] with the 32x32 MFMA (bf16: v_mfma_f32_32x32x16_bf16; fp32: 4 x
// v_mfma_f32_32x32x2f32 per 8-wide k group; FP8 E4M3 with power-of-two row scales:
// v_mfma_scale_f32_32x32x64_f8f6f4, the scales applied by the instruction itself). Waves sit in a
// 2 (m) x 4 (n) grid; each owns a 128 x 64 sub-tile = 4 x 2 MFMA blocks = 128 accumulator
// registers per lane.
//
// Operands are staged through LDS, 128 bytes of K per row per stage (64 bf16 / 32 fp32 / 128 fp8),
// in two stages. Dense operands go global -> LDS directly (buffer_load_dwordx4 ... lds): each wave
// instruction fills 1 KiB of LDS, lane l writing bytes [16 l, 16 l + 16), and the buffer
// descriptor's range check returns zeros past the operand's last valid row, so tails need no VALU
// work and loads need no staging registers; a step's direct loads go out one per MFMA of the group
// after the barrier. 4-bit weights take a register path that dequantises on the way into LDS,
// loaded steps ahead into two register sets and dequantised between the MFMAs (gemm_run_q4k,
// gemm_run_q4n). Within a K step the fragments of K group g + 1 are read while group g's MFMAs run
// (one read between consecutive MFMAs, pinned with sched_group_barrier); for K-major x K-major
// stages the step's barrier sits before its last K group (gemm_step), for the others at its end
// (gemm_step_end).
//
// Each operand tile keeps its global orientation in LDS, unpadded and XOR-swizzled per 16-byte
// chunk (chunk c of row r is stored at chunk c ^ swz(r)):
//   K-major  ([rows][k], k contiguous):   [256 rows][128 B], swz = (r >> 1) & 7 (fp8: r & 6);
//                                          fragments via ds_read_b128.
//   MN-major ([k][cols], cols contiguous): bf16 [64 rows][512 B], swz = 10 (r & 3);
//                                          fragments via the transposing ds_read_b64_tr_b16.
//                                          fp32 [32 rows][1024 B], swz = 8 ((r >> 2) & 1);
//                                          fragments via 4 scalar reads.
// The swizzles keep both the 16-byte fragment reads and the transposing reads on distinct banks.
// So the forward (A = W, B = h, both K-major), the dh GEMM (A = coeff K-major, B = W N-major) and
// the dW GEMM (A = coeff M-major, B = h N-major) run on one engine with no transposed copy in HBM.
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kTile = 256;                  // tile extent in m and n
constexpr int kKBytes = 128;                // bytes of K per stage per row
constexpr int kStageBytes = 32768;          // LDS bytes of one operand stage
constexpr int kLdsBytes = 4 * kStageBytes;  // A and B, two stages each
constexpr uint32_t kBufferFlags = 0x00020000u;   // raw buffer descriptor word 3 (32-bit data format)

// LDS swizzles (16-byte chunk index XOR a function of the row). K-major: row r's chunk c sits at
// c ^ ((r >> 1) & 7). gfx950's LDS has 64 four-byte banks and serves 16 lanes of a ds_read_b128 per
// cycle: 16 consecutive 128-byte rows, two to a 256-byte bank row, so each pair of rows must take
// one of 8 distinct chunk positions (a swizzle of r & 7 repeats after 8 rows and makes every read
// a 2-way bank conflict). Rows 32 apart share the swizzle (a fragment's 32-row blocks are constant
// offsets apart).
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_mn16(int r) { return 10 * (r & 3); }
__device__ __forceinline__ int swz_mn32(int r) { return ((r >> 2) & 1) << 3; }

// Wait until this wave's outstanding vector-memory operations (including LDS-direct loads) are done.
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same wait as an instruction the compiler's wait insertion sees (s_waitcnt immediate on gfx9:
// vmcnt bits [3:0] and [15:14] zero, expcnt 7 and lgkmcnt 15, i.e. not waited on): register loads
// issued before it then count as complete, so the compiler adds no later wait for them (the 4-bit
// loops read such loads' registers a step after the barrier that waited for them).
__device__ __forceinline__ void vm_wait_seen() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(uint32_t)n, (int)kBufferFlags);
}

// ------------------------------------------------------------------------------------------
// Element policies: K per stage, K groups per stage, fragment reads and the MFMA step. A fragment
// holds, for the 32-row block starting at row0, row row0 + l % 32 in lane l and a fixed set of k
// slots of K group kg: 16 bytes per lane for bf16 (kg*16 + (l / 32) * 8 + [0, 8)) and fp32
// (kg*8 + (l / 32) * 4 + [0, 4)), 32 bytes for fp8 (kg*64 + (l / 32) * 32 + [0, 32)). Any
// consistent k-slot assignment gives the same sum, as long as A and B use the same one.
// Scales: the per-row scale operands of the MFMA (an empty type where the format has none).
// ------------------------------------------------------------------------------------------
struct NoScales {};

struct EBf16 {
  typedef __bf16 T;
  typedef bf16x8 Frag;
  typedef NoScales Scales;
  static constexpr int kSize = 2;
  static constexpr int kBK = 64;           // K elements per stage
  static constexpr int kGroups = 4;        // MFMA K groups per stage
  static constexpr int kReadsK = 1;        // LDS reads per K-major fragment
  static constexpr int kSets = 2;          // fragment register sets (2: next group read ahead)
  static constexpr int kSwzShift = 1;      // K-major swizzle (r >> kSwzShift) & kSwzK (swz_k)
  static constexpr int kSwzK = 7;
  static constexpr int kMnRows = 64;       // rows of an MN-major stage
  static constexpr int kMnChunks = 32;     // 16-byte chunks per MN-major row

  static __device__ __forceinline__ Frag frag_k(const char* s, int row0, int kg, int l) {
    const int r = row0 + (l & 31), c = kg * 2 + (l >> 5);
    return *(const Frag*)(s + r * kKBytes + ((c ^ swz_k(r)) << 4));
  }
  // Transposing read: within each 16-lane group, source lane q reads 4 contiguous columns of row
  // (k0 + q/4); the hardware hands output lane j, slot i the element j%4 of source lane 4i + j/4,
  // i.e. column j of row k0 + i. Two reads (rows k0..k0+3 and k0+4..k0+7) give the lane's 8 k slots.
  static __device__ __forceinline__ Frag frag_mn(const char* s, int col0, int kg, int l) {
    const int g = l >> 4, q = l & 15;
    const int row = kg * 16 + 8 * (g >> 1) + (q >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (q & 3);
    const char* p = s + row * (kMnChunks * 16) + (((col >> 3) ^ swz_mn16(row)) << 4) + (col & 7) * 2;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * kMnChunks * 16));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(Frag, v);
  }
  template <int MB, int NB>
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b, const Scales&) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

struct EF32 {
  typedef float T;
  typedef f32x4 Frag;
  typedef NoScales Scales;
  static constexpr int kSize = 4;
  static constexpr int kBK = 32;
  static constexpr int kGroups = 4;
  static constexpr int kReadsK = 1;
  static constexpr int kSets = 2;
  static constexpr int kSwzShift = 1;
  static constexpr int kSwzK = 7;
  static constexpr int kMnRows = 32;
  static constexpr int kMnChunks = 64;

  static __device__ __forceinline__ Frag frag_k(const char* s, int row0, int kg, int l) {
    const int r = row0 + (l & 31), c = kg * 2 + (l >> 5);
    return *(const Frag*)(s + r * kKBytes + ((c ^ swz_k(r)) << 4));
  }
  static __device__ __forceinline__ Frag frag_mn(const char* s, int col0, int kg, int l) {
    const int row = kg * 8 + (l >> 5) * 4;        // rows row .. row+3 share one swizzle
    const int col = col0 + (l & 31);
    const char* p = s + row * (kMnChunks * 16) + (((col >> 2) ^ swz_mn32(row)) << 4) + (col & 3) * 4;
    Frag f;
    f[0] = *(const float*)(p);
    f[1] = *(const float*)(p + kMnChunks * 16);
    f[2] = *(const float*)(p + 2 * kMnChunks * 16);
    f[3] = *(const float*)(p + 3 * kMnChunks * 16);
    return f;
  }
  template <int MB, int NB>
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b, const Scales&) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  }
};

// FP8 E4M3 operands (K-major only: the logit GEMMs) with one power-of-two scale per row, given as
// E8M0 exponent bytes. Scales.a holds the exponents of the lane's row in the wave's four 32-row
// A blocks (byte mb), Scales.b those of its two B blocks (byte nb); the MFMA's byte selects pick
// them, so C accumulates 2^(ea + eb) sum_k a_k b_k with exact products in fp32.
struct EFp8 {
  typedef uint8_t T;
  typedef i32x8 Frag;
  struct Scales {
    int32_t a, b;
  };
  static constexpr int kSize = 1;
  static constexpr int kBK = 128;
  static constexpr int kGroups = 2;
  static constexpr int kReadsK = 2;
  // One register set: 32-byte fragments in two sets (96 VGPRs) and the 128 accumulators would
  // not fit in a wave's 256 registers. A group's reads follow its MFMAs; the SIMD's other wave
  // covers their latency.
  static constexpr int kSets = 1;
  // Swizzle r & 6: an even XOR keeps a fragment's two chunks (c even, c + 1) adjacent, so both
  // reads share one address register (offsets 0 and 16). A 128-byte row has only four such chunk
  // pairs, so 16 lanes of one read meet a 2-way bank conflict either way.
  static constexpr int kSwzShift = 0;
  static constexpr int kSwzK = 6;

  static __device__ __forceinline__ Frag frag_k(const char* s, int row0, int kg, int l) {
    const int r = row0 + (l & 31), c = (kg * 4 + (l >> 5) * 2) ^ (r & kSwzK);
    const i32x4 lo = *(const i32x4*)(s + r * kKBytes + (c << 4));
    const i32x4 hi = *(const i32x4*)(s + r * kKBytes + (c << 4) + 16);
    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  template <int MB, int NB>
  static __device__ __forceinline__ void mma(f32x16& c, const Frag& a, const Frag& b, const Scales& sc) {
    // Format selectors 0 / 0: both operands FP8 E4M3.
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, MB, sc.a, NB, sc.b);
  }
};

// One direct global -> LDS load: 16 bytes per lane from byte voff + soff of the descriptor's range,
// lane l's data landing at LDS byte (lds + 16 l); bytes past the range read as zero.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char* lds, uint32_t voff,
                                      uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// ------------------------------------------------------------------------------------------
// Dense loaders: global -> LDS directly. A stage is 2048 chunks of 16 bytes; wave w issues
// instructions i = 0..3 filling LDS bytes [(4w + i) KiB, +1 KiB), lane l the chunk 64 (4w + i) + l.
// ------------------------------------------------------------------------------------------

// K-major operand: rows [row0, row0 + 256) of a row-major matrix, bytes [kb, kb + 128) of each row,
// chunk c of row r stored at chunk c ^ ((r >> kShift) & kSwzMask).
template <int kShift, int kSwzMask>
struct DmaKS {
  const char* base;
  int64_t ld, n_rows;
  uint32_t voff[4];
  int wave_lds;                   // this wave's 4 KiB of a stage (uniform: an SGPR)
  __amdgpu_buffer_rsrc_t rs;
  __device__ __forceinline__ void init(const void* b, int64_t ld_bytes, int64_t rows) {
    base = (const char*)b;
    ld = ld_bytes;
    n_rows = rows;
    wave_lds = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) * 4096);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = (4 * w + i) * 64 + l;
      const int r = j >> 3, c = (j & 7) ^ ((r >> kShift) & kSwzMask);
      voff[i] = (uint32_t)(r * ld_bytes + c * 16);
    }
  }
  // The descriptor covers whole rows [row0, n_rows) and depends on the tile only; the K offset kb
  // (within a row) goes in the scalar offset. A row past n_rows starts past the range, so all of it
  // reads as zero.
  __device__ __forceinline__ void issue(int64_t row0, int64_t kb, char* stage) {
    rs = make_rsrc(base + row0 * ld, (n_rows - row0) * ld);   // branch-free: see gemm_step
    char* s = stage + wave_lds;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rs, s + i * 1024, voff[i], (uint32_t)kb);
  }
  __device__ __forceinline__ void commit(char*) const {}
};
typedef DmaKS<1, 7> DmaK;   // swz_k

// MN-major operand: rows [k0, k0 + kMnRows) of a row-major matrix of n_rows rows, bytes
// [cb, cb + kMnChunks*16). The descriptor starts at column byte cb of row 0 and ends n_rows rows
// later (it depends on the column block only); the row offset k0 ld goes in the per-lane offset,
// so a row at or past n_rows lies past the range and reads as zero. Callers pass the matrix from
// the first row they use, so that n_rows ld stays within 32 bits.
template <class E>
struct DmaMN {
  const char* base;
  int64_t ld, n_rows;
  uint32_t voff[4];
  int wave_lds;                   // this wave's 4 KiB of a stage (uniform: an SGPR)
  __device__ __forceinline__ void init(const void* b, int64_t ld_bytes, int64_t rows) {
    base = (const char*)b;
    ld = ld_bytes;
    n_rows = rows;
    wave_lds = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) * 4096);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = (4 * w + i) * 64 + l;
      const int r = j / E::kMnChunks, p = j % E::kMnChunks;
      const int c = p ^ (E::kSize == 2 ? swz_mn16(r) : swz_mn32(r));
      voff[i] = (uint32_t)(r * ld_bytes + c * 16);
    }
  }
  __device__ __forceinline__ void issue(int64_t k0, int64_t cb, char* stage) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + cb, n_rows * ld - cb);
    const uint32_t ro = (uint32_t)(k0 * ld);
    char* s = stage + wave_lds;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rs, s + i * 1024, voff[i] + ro);
  }
  __device__ __forceinline__ void commit(char*) const {}
};

// ------------------------------------------------------------------------------------------
// 4-bit weights: global -> registers -> dequantise -> LDS.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (lo in the low half), each rounded to nearest even: one
// v_cvt_pk_bf16_f32 (converting the halves one at a time costs two of them plus a shift and an or).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 codes of one packed word -> 8 bf16 (16 bytes): w = scale * q + bias in fp32, then RNE. The
// even and odd codes are masked into the four bytes of two words, which the byte-to-float
// conversions (v_cvt_f32_ubyte0..3) read directly.
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, float scale, float bias) {
  uint32_t even = w & 0x0F0F0F0Fu;                 // codes 0, 2, 4, 6
  uint32_t odd = (w >> 4) & 0x0F0F0F0Fu;           // codes 1, 3, 5, 7
  // Opaque to the compiler, which would otherwise fold the masks into one bit-field extract per
  // code: each byte then converts in one instruction (v_cvt_f32_ubyte0..3).
  asm("" : "+v"(even));
  asm("" : "+v"(odd));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float q0 = (float)((even >> (8 * i)) & 0xFFu);
    const float q1 = (float)((odd >> (8 * i)) & 0xFFu);
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

// 4-bit weights as a K-major operand (gemm_run_q4k): 256 vocabulary rows x 64 codes (one group) per
// stage; thread tid owns row tid / 2, codes [32 (tid % 2), +32) = chunks 4 (tid % 2) + w. The words
// of a step are loaded three steps ahead into register set S and dequantised into LDS during the
// step before their use, interleaved with that step's MFMAs. Rows past the vocabulary read row 0 (in
// bounds) and are zeroed at commit; callers keep k0 inside the row.
struct Q4K2 {
  Q4Weight W;
  u32x4 q[2];
  // bf16 bits of the group's scale and bias, each in a register of its own: nothing combines
  // them before the commit, so no ALU op waits on these loads where they are issued.
  uint16_t sbits[2], bbits[2];
  bool ok[2];
  static constexpr int kLoads = 3;   // vector-memory loads per issue: the words, scale, bias
  __device__ __forceinline__ void init(const Q4Weight& w) { W = w; }
  // live = false stages zeros (the words are still read, from row0's group at k0, in bounds).
  template <int S>
  __device__ __forceinline__ void issue(int64_t row0, int64_t k0, bool live) {
    const int tid = threadIdx.x;
    const int64_t gr = row0 + (tid >> 1);
    const bool in = gr < W.V && live;
    const int64_t r = in ? gr : 0;
    q[S] = *(const u32x4*)(W.wq + r * (W.d >> 3) + (k0 >> 3) + (tid & 1) * 4);
    const int64_t gi = r * (W.d >> 6) + (k0 >> 6);
    sbits[S] = W.scales[gi];
    bbits[S] = W.biases[gi];
    ok[S] = in;
  }
  // Writes [W0, W1) of set S into the stage, one 16-byte LDS write (8 codes) each. Write w of a
  // lane in an odd row stores its word (w + 2) & 3, of one in an even row its word w: the 16 lanes
  // an LDS write serves together then cover 16 different 16-byte bank slots (measured: 105 bytes per
  // clock per CU, against 85 with every lane storing word w).
  template <int S, int W0, int W1>
  __device__ __forceinline__ void commit_words(char* stage) const {
    const int tid = threadIdx.x, r = tid >> 1;
    const bool odd = r & 1;
    const float scale = ok[S] ? bf16_bits_to_f32(sbits[S]) : 0.f;
    const float bias = ok[S] ? bf16_bits_to_f32(bbits[S]) : 0.f;
    char* row = stage + r * kKBytes;
#pragma unroll
    for (int w = W0; w < W1; ++w) {
      const int ww = odd ? (w + 2) & 3 : w;
      const uint32_t word = odd ? q[S][(w + 2) & 3] : q[S][w];
      *(u32x4*)(row + (((tid & 1) * 4 + ww) ^ swz_k(r)) * 16) = dequant_word(word, scale, bias);
    }
  }
  template <int S>
  __device__ __forceinline__ void commit(char* stage) const { commit_words<S, 0, 4>(stage); }
};

// 4-bit weights as an N-major operand (gemm_run_q4n; rows = vocabulary = k, columns = hidden = n):
// 64 rows x 256 codes per stage; thread tid owns row tid / 8, codes [32 (tid % 8), +32) = chunks
// 4 (tid % 8) + w. The words of a step are loaded two steps ahead into register set S and
// dequantised into LDS during the step before their use, interleaved with its MFMAs. live = false
// stages zeros.
struct Q4N2 {
  Q4Weight W;
  int64_t v_end;             // rows >= v_end read as zero
  u32x4 q[2];
  uint16_t sbits[2], bbits[2];   // bf16 bits of the group's scale and bias, separate registers
  bool ok[2];
  static constexpr int kLoads = 3;   // vector-memory loads per issue: the words, scale, bias
  __device__ __forceinline__ void init(const Q4Weight& w, int64_t vend) { W = w; v_end = vend; }
  template <int S>
  __device__ __forceinline__ void issue(int64_t k0, int64_t n0, bool live) {
    const int tid = threadIdx.x;
    const int64_t gr = k0 + (tid >> 3);
    const int64_t gc = n0 + (tid & 7) * 32;
    const bool in = live && gr < v_end && gc < W.d;
    const int64_t r = in ? gr : 0, c = in ? gc : 0;
    q[S] = *(const u32x4*)(W.wq + r * (W.d >> 3) + (c >> 3));
    const int64_t gi = r * (W.d >> 6) + (c >> 6);
    sbits[S] = W.scales[gi];
    bbits[S] = W.biases[gi];
    ok[S] = in;
  }
  // Writes [W0, W1) of set S into the stage, one 16-byte LDS write (8 codes) each. Write w of lane
  // j (of the 8 on a row) stores its word (w + j / 2) & 3: the 16 lanes an LDS write serves
  // together then cover 16 different 16-byte bank slots (measured: 105 bytes per clock per CU,
  // against 43 with every lane storing word w).
  template <int S, int W0, int W1>
  __device__ __forceinline__ void commit_words(char* stage) const {
    const int tid = threadIdx.x, r = tid >> 3, k = (tid >> 1) & 3;
    const float scale = ok[S] ? bf16_bits_to_f32(sbits[S]) : 0.f;
    const float bias = ok[S] ? bf16_bits_to_f32(bbits[S]) : 0.f;
    char* row = stage + r * (EBf16::kMnChunks * 16);
#pragma unroll
    for (int w = W0; w < W1; ++w) {
      const int ww = (w + k) & 3;
      const uint32_t lo = (k & 1) ? q[S][(w + 1) & 3] : q[S][w];
      const uint32_t hi = (k & 1) ? q[S][(w + 3) & 3] : q[S][(w + 2) & 3];
      const uint32_t word = (k & 2) ? hi : lo;
      *(u32x4*)(row + (((tid & 7) * 4 + ww) ^ swz_mn16(r)) * 16) = dequant_word(word, scale, bias);
    }
  }
};

// ------------------------------------------------------------------------------------------
// Compute one LDS stage into the wave's 4 x 2 accumulator blocks.
// ------------------------------------------------------------------------------------------
template <class E, bool K>
__device__ __forceinline__ typename E::Frag frag(const char* s, int row0, int kg, int l) {
  if constexpr (K) return E::frag_k(s, row0, kg, l);
  else return E::frag_mn(s, row0, kg, l);
}

template <class E, bool AK, bool BK>
__device__ __forceinline__ void load_frags(const char* sa, const char* sb, int kg, int wm, int wn,
                                           int l, typename E::Frag (&a)[4],
                                           typename E::Frag (&b)[2]) {
  // In the order the MFMAs consume them: b0, a0, b1, then a1..a3.
  b[0] = frag<E, BK>(sb, wn * 64, kg, l);
  a[0] = frag<E, AK>(sa, wm * 128, kg, l);
  b[1] = frag<E, BK>(sb, wn * 64 + 32, kg, l);
#pragma unroll
  for (int mb = 1; mb < 4; ++mb) a[mb] = frag<E, AK>(sa, wm * 128 + mb * 32, kg, l);
}

// Instruction counts of one K group, for the scheduling pattern below: LDS reads per fragment
// (ds_read_b128s for K-major: one, or two for fp8; two transposing reads (bf16) or four dword
// reads (fp32) for MN-major) and MFMA instructions per fragment pair.
template <class E, bool K>
constexpr int reads_per_frag() { return K ? E::kReadsK : (E::kSize == 2 ? 2 : 4); }
template <class E>
constexpr int mfma_per_mma() { return E::kSize == 2 ? 1 : 4; }

// The MFMAs of one K group: the wave's 4 x 2 blocks of 32 x 32, in the order (0,0), (0,1), (1,0),
// ... (block indices are template arguments: the fp8 MFMA takes its scale byte selects as
// constants).
template <class E, int MB = 0, int NB = 0>
__device__ __forceinline__ void mma_group(f32x16 (&acc)[4][2], const typename E::Frag (&a)[4],
                                          const typename E::Frag (&b)[2],
                                          const typename E::Scales& sc) {
  E::template mma<MB, NB>(acc[MB][NB], a[MB], b[NB], sc);
  if constexpr (NB + 1 < 2) mma_group<E, MB, NB + 1>(acc, a, b, sc);
  else if constexpr (MB + 1 < 4) mma_group<E, MB + 1, 0>(acc, a, b, sc);
}

// Pins the order of the LDS reads and MFMAs of kGroups K groups, each group's MFMAs interleaved
// with the reads of the group after it, spread over the first three quarters of the MFMAs so that
// the last read has a few MFMAs' time to land before its group starts.
template <class E, bool AK, bool BK, int kGroups>
__device__ __forceinline__ void sched_groups() {
  constexpr int kReads = 4 * reads_per_frag<E, AK>() + 2 * reads_per_frag<E, BK>();
  constexpr int kMfma = 8 * mfma_per_mma<E>();
  constexpr int kSpan = kMfma * 3 / 4;
  static_assert(kReads <= 2 * kSpan, "at most two reads between MFMAs");
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int n = i < kSpan ? (i + 1) * kReads / kSpan - i * kReads / kSpan : 0;
      if (n == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (n == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
}

// The post-barrier region of a K-major step: one K group's MFMAs, the next stage's first-group
// reads after the first ones, and one direct load (VMEM read) after each MFMA.
template <class E, bool AK, bool BK>
__device__ __forceinline__ void sched_groups_loads() {
  constexpr int kReads = 4 * reads_per_frag<E, AK>() + 2 * reads_per_frag<E, BK>();
  constexpr int kMfma = 8 * mfma_per_mma<E>();
  constexpr int kSpan = kMfma * 3 / 4;
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const int n = i < kSpan ? (i + 1) * kReads / kSpan - i * kReads / kSpan : 0;
    if (n == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (n == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// Row scales fetched before a step's wait are taken here, right after it: the compiler then counts
// their loads as done at this point and does not place its own wait for them after the next
// step's direct loads are issued (which would make the fragment reads wait for those loads).
__device__ __forceinline__ void hold_scales(NoScales&) {}
template <class S>
__device__ __forceinline__ void hold_scales(S& sc) {
  asm volatile("" : "+v"(sc.a), "+v"(sc.b));
}

// An empty asm that reads and "writes" the accumulators: the MFMAs before it stay before it.
__device__ __forceinline__ void hold_acc(f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) asm volatile("" : "+v"(acc[mb][nb]));
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
}

// LDS of the engine: four distinct objects (A and B, two stages each), so that the compiler can
// tell a stage being filled by direct loads from the stage being read and does not make the reads
// wait for the in-flight loads.
struct Smem {
  char* a0;
  char* a1;
  char* b0;
  char* b1;
};
#define ORPO_DECLARE_SMEM(name)                                        \
  __shared__ __attribute__((aligned(1024))) char name##_a0[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char name##_a1[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char name##_b0[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char name##_b1[kStageBytes]; \
  const Smem name = {name##_a0, name##_a1, name##_b0, name##_b1}

// Fragments of E::kSets K groups: group kg lives in set kg % kSets.
template <class E>
struct FragSets {
  typename E::Frag a[E::kSets][4], b[E::kSets][2];
};

// One K group with streamed fragments (policies with one fragment set), in two parts. The group's
// B pair and first A block are in f on entry. group_head reads A blocks 1..3 of group kg of stage
// sa, each under the two MFMAs of the block before, and returns block 3; group_tail reads the next
// group's B pair and first A block (group nkg of stage (nsa, nsb)) under the last two MFMAs. At
// most six fragments are live at once and each read has two MFMAs to land. The stage's workgroup
// barrier goes between the last group's head and tail: every read of the stage is then done, and
// the last two MFMAs overlap the next stage's first reads.
template <class E, bool AK, bool BK>
__device__ __forceinline__ typename E::Frag group_head(f32x16 (&acc)[4][2], const FragSets<E>& f,
                                                       const char* __restrict__ sa, int kg,
                                                       const typename E::Scales& sc, int wm, int l) {
  constexpr int kR = reads_per_frag<E, AK>();
  const typename E::Frag a1 = frag<E, AK>(sa, wm * 128 + 32, kg, l);
  E::template mma<0, 0>(acc[0][0], f.a[0][0], f.b[0][0], sc);
  E::template mma<0, 1>(acc[0][1], f.a[0][0], f.b[0][1], sc);
  const typename E::Frag a2 = frag<E, AK>(sa, wm * 128 + 64, kg, l);
  E::template mma<1, 0>(acc[1][0], a1, f.b[0][0], sc);
  E::template mma<1, 1>(acc[1][1], a1, f.b[0][1], sc);
  const typename E::Frag a3 = frag<E, AK>(sa, wm * 128 + 96, kg, l);
  E::template mma<2, 0>(acc[2][0], a2, f.b[0][0], sc);
  E::template mma<2, 1>(acc[2][1], a2, f.b[0][1], sc);
  __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  return a3;
}

template <class E, bool AK, bool BK>
__device__ __forceinline__ void group_tail(f32x16 (&acc)[4][2], FragSets<E>& f,
                                           const typename E::Frag& a3, const char* __restrict__ nsa,
                                           const char* __restrict__ nsb, int nkg,
                                           const typename E::Scales& sc, int wm, int wn, int l) {
  constexpr int kR = reads_per_frag<E, AK>(), kRb = reads_per_frag<E, BK>();
  const typename E::Frag nb0 = frag<E, BK>(nsb, wn * 64, nkg, l);
  const typename E::Frag na0 = frag<E, AK>(nsa, wm * 128, nkg, l);
  const typename E::Frag nb1 = frag<E, BK>(nsb, wn * 64 + 32, nkg, l);
  E::template mma<3, 0>(acc[3][0], a3, f.b[0][0], sc);
  E::template mma<3, 1>(acc[3][1], a3, f.b[0][1], sc);
  f.a[0][0] = na0;
  f.b[0][0] = nb0;
  f.b[0][1] = nb1;
  __builtin_amdgcn_sched_group_barrier(0x100, kR + 2 * kRb, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
}

// One K step s, reading stage (ca, cb); stage (na, nb) holds step s + 1. The workgroup barrier
// sits before the last K group rather than at the end of the step: by then every wave holds that
// group's fragments in registers, so its MFMAs run while the next stage's first fragments are read,
// and the MFMA pipe does not idle on an LDS round trip after each barrier.
//   region 1: MFMAs of groups 0..G-2, each with the next group's reads (G = E::kGroups);
//   barrier:  this stage is no longer read by anyone, stage s + 1 is in LDS (own loads waited
//             first, register-staged loads committed first); the loads of step s + 2 then go into
//             this stage;
//   region 2: MFMAs of group G-1 with the reads of step s + 1's group 0 (issued unconditionally; on
//             the last step they read a stale stage and are never used), then the epilogue if the
//             step ends a tile.
// Row scales (fp8): the last step of each tile fetches the next tile's scales (`scales(tile)`)
// just before its wait for the step's loads, so they cost no wait of their own; they replace the
// current ones after the tile's epilogue.
// Step positions, counted without division: `cur` is step s (tile, K step), `ahead` step s + 2.
struct StepPos {
  int tile, ks;
  __device__ __forceinline__ void next(int nk) {
    if (++ks == nk) {
      ks = 0;
      ++tile;
    }
  }
};

template <class E, bool AK, bool BK, bool kClear, bool kDmaOnly, class Issue, class Commit,
          class Epi, class Scl>
__device__ __forceinline__ void gemm_step(int s, int total, int nk, StepPos& cur, StepPos& ahead,
                                          char* __restrict__ ca,
                                          char* __restrict__ cb, char* __restrict__ na,
                                          char* __restrict__ nb, Issue& issue, Commit& commit,
                                          Epi& epi, Scl& scales, typename E::Scales& sc,
                                          typename E::Scales& sc_next, FragSets<E>& f,
                                          f32x16 (&acc)[4][2], int wm, int wn, int l) {
  constexpr int kG = E::kGroups;
  typename E::Frag a_last;   // streamed path: the last group's A block 3, across the barrier
  if constexpr (E::kSets == 2) {
#pragma unroll
    for (int kg = 0; kg < kG - 1; ++kg) {
      load_frags<E, AK, BK>(ca, cb, kg + 1, wm, wn, l, f.a[(kg + 1) & 1], f.b[(kg + 1) & 1]);
      mma_group<E>(acc, f.a[kg & 1], f.b[kg & 1], sc);
    }
    sched_groups<E, AK, BK, kG - 1>();
  } else {
    // Streamed fragments: whole groups, then the last group's head; its tail follows the barrier.
    // The MFMAs may not move below the barrier (an empty asm takes the accumulators here), where
    // they would hold more fragments live.
#pragma unroll
    for (int kg = 0; kg < kG - 1; ++kg) {
      const typename E::Frag a3 = group_head<E, AK, BK>(acc, f, ca, kg, sc, wm, l);
      group_tail<E, AK, BK>(acc, f, a3, ca, cb, kg + 1, sc, wm, wn, l);
    }
    a_last = group_head<E, AK, BK>(acc, f, ca, kG - 1, sc, wm, l);
    hold_acc(acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  const bool ends_tile = cur.ks == nk - 1;
  if (s + 1 < total) commit(na, nb);
  if (ends_tile && s + 1 < total) sc_next = scales(cur.tile + 1);
  vm_wait();
  hold_scales(sc_next);
  __syncthreads();
  if constexpr (E::kSets == 2 && kDmaOnly) {
    // The loads of step s + 2 go out one after each MFMA of this region instead of as one burst
    // of every wave after the barrier. They are issued unconditionally so that they share the
    // MFMAs' basic block: only for direct loads through buffer descriptors, which past the last
    // step read zeros or bytes inside the operand's range into a stage that is never read again.
    issue(ahead.tile, ahead.ks, ca, cb);
    ahead.next(nk);
    load_frags<E, AK, BK>(na, nb, 0, wm, wn, l, f.a[0], f.b[0]);
    mma_group<E>(acc, f.a[(kG - 1) & 1], f.b[(kG - 1) & 1], sc);
    sched_groups_loads<E, AK, BK>();
  } else if constexpr (E::kSets == 2) {
    if (s + 2 < total) issue(ahead.tile, ahead.ks, ca, cb);
    ahead.next(nk);
    load_frags<E, AK, BK>(na, nb, 0, wm, wn, l, f.a[0], f.b[0]);
    mma_group<E>(acc, f.a[(kG - 1) & 1], f.b[(kG - 1) & 1], sc);
    sched_groups<E, AK, BK, 1>();
  } else {
    if (s + 2 < total) issue(ahead.tile, ahead.ks, ca, cb);
    ahead.next(nk);
    group_tail<E, AK, BK>(acc, f, a_last, na, nb, 0, sc, wm, wn, l);
  }
  if (ends_tile) {
    epi(cur.tile, acc);
    if (kClear) zero_acc(acc);
    sc = sc_next;
  }
  cur.next(nk);
}

// One K step with the barrier at its end, for stages read with transposing instructions (there the
// barrier before the last group measured slower): the next step's loads are issued first, then the
// MFMAs of the four groups with each group's reads one group ahead (left to the compiler's
// schedule), then the step's epilogue, wait and barrier.
template <class E, bool AK, bool BK, bool kClear, bool kDmaOnly, class Issue, class Commit,
          class Epi, class Scl>
__device__ __forceinline__ void gemm_step_end(int s, int total, int nk, StepPos& cur,
                                              StepPos& ahead, char* __restrict__ ca,
                                              char* __restrict__ cb, char* __restrict__ na,
                                              char* __restrict__ nb, Issue& issue, Commit& commit,
                                              Epi& epi, Scl& scales, typename E::Scales& sc,
                                              typename E::Scales& sc_next, f32x16 (&acc)[4][2],
                                              int wm, int wn, int l) {
  constexpr int kG = E::kGroups;
  // ahead = step s + 1 here. Direct loads only: issued unconditionally (as in gemm_step) and
  // pinned one after each of the step's first MFMAs rather than as one burst before them.
  if constexpr (kDmaOnly) issue(ahead.tile, ahead.ks, na, nb);
  else if (s + 1 < total) issue(ahead.tile, ahead.ks, na, nb);
  ahead.next(nk);
  static_assert(E::kSets == 2, "transposing stages read the next group ahead");
  FragSets<E> f;
  load_frags<E, AK, BK>(ca, cb, 0, wm, wn, l, f.a[0], f.b[0]);
#pragma unroll
  for (int kg = 0; kg < kG; ++kg) {
    if (kg + 1 < kG)
      load_frags<E, AK, BK>(ca, cb, kg + 1, wm, wn, l, f.a[(kg + 1) & 1], f.b[(kg + 1) & 1]);
    mma_group<E>(acc, f.a[kg & 1], f.b[kg & 1], sc);
  }
  if constexpr (kDmaOnly) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  }
  const bool ends_tile = cur.ks == nk - 1;
  if (s + 1 < total) commit(na, nb);
  if (ends_tile && s + 1 < total) sc_next = scales(cur.tile + 1);
  if (ends_tile) {
    epi(cur.tile, acc);
    if (kClear) zero_acc(acc);
    sc = sc_next;
  }
  cur.next(nk);
  vm_wait();
  __syncthreads();
}

// The main loop over n_tiles consecutive output tiles of nk K steps each (step s is K step s % nk
// of tile s / nk).
//   issue(tile, ks, stageA, stageB): start the loads of step (tile, ks) into the given stages;
//   commit(stageA, stageB): finish register-staged loads into LDS (no-op for direct loads);
//   epi(tile, acc): runs after the tile's last K step (it must not touch LDS), then the
//   accumulators are cleared unless kClear is false (single-tile callers read acc after the loop);
//   scales(tile): the MFMA row scales of a tile (fp8; gemm_run passes none for other formats).
// Two stages: step s + 1's loads are in flight during step s's MFMAs. The loop is unrolled by two
// so that every step reads and fills statically known stages.
template <class E, bool AK, bool BK, bool kClear = true, bool kDmaOnly = false, class Issue,
          class Commit, class Epi, class Scl>
__device__ __forceinline__ void gemm_run_scaled(const Smem& sm, int n_tiles, int nk, Issue&& issue,
                                                Commit&& commit, Epi&& epi, Scl&& scales,
                                                f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int total = n_tiles * nk;
  if (total <= 0) return;
  typename E::Scales sc = scales(0), sc_next = sc;
  StepPos cur{0, 0}, ahead{0, 0};
  issue(0, 0, sm.a0, sm.b0);
  ahead.next(nk);
  commit(sm.a0, sm.b0);
  vm_wait();
  __syncthreads();
  if constexpr (!(AK && BK)) {
    // Transposing reads: barrier at the end of each step; `ahead` runs one step ahead.
    for (int it = 0; it < total; it += 2) {
      gemm_step_end<E, AK, BK, kClear, kDmaOnly>(it, total, nk, cur, ahead, sm.a0, sm.b0, sm.a1,
                                                 sm.b1, issue, commit, epi, scales, sc, sc_next,
                                                 acc, wm, wn, l);
      if (it + 1 < total)
        gemm_step_end<E, AK, BK, kClear, kDmaOnly>(it + 1, total, nk, cur, ahead, sm.a1, sm.b1,
                                                   sm.a0, sm.b0, issue, commit, epi, scales, sc,
                                                   sc_next, acc, wm, wn, l);
    }
    vm_wait();   // the loads past the last step
    return;
  }
  // K-major stages: `ahead` runs two steps ahead.
  if (total > 1) issue(ahead.tile, ahead.ks, sm.a1, sm.b1);
  ahead.next(nk);
  FragSets<E> f;
  load_frags<E, AK, BK>(sm.a0, sm.b0, 0, wm, wn, l, f.a[0], f.b[0]);
  for (int it = 0; it < total; it += 2) {
    gemm_step<E, AK, BK, kClear, kDmaOnly>(it, total, nk, cur, ahead, sm.a0, sm.b0, sm.a1, sm.b1,
                                           issue, commit, epi, scales, sc, sc_next, f, acc, wm,
                                           wn, l);
    if (it + 1 < total)
      gemm_step<E, AK, BK, kClear, kDmaOnly>(it + 1, total, nk, cur, ahead, sm.a1, sm.b1, sm.a0,
                                             sm.b0, issue, commit, epi, scales, sc, sc_next, f,
                                             acc, wm, wn, l);
  }
  vm_wait();   // the loads past the last step, before the caller reuses the LDS
}

template <class E, bool AK, bool BK, bool kClear = true, bool kDmaOnly = false, class Issue,
          class Commit, class Epi>
__device__ __forceinline__ void gemm_run(const Smem& sm, int n_tiles, int nk, Issue&& issue,
                                         Commit&& commit, Epi&& epi, f32x16 (&acc)[4][2]) {
  gemm_run_scaled<E, AK, BK, kClear, kDmaOnly>(sm, n_tiles, nk, issue, commit, epi,
                                               [](int) { return typename E::Scales{}; }, acc);
}

// ------------------------------------------------------------------------------------------
// The 4-bit head's K-major loop (forward and coefficient tiles, A = the 4-bit weights, B dense).
// The two-stage schedule of gemm_step with the A operand one step further ahead: after step s's
// barrier B's direct loads of step s + 2 are issued, then (in a scheduling region of their own, so
// that they come after them) the words of step s + 3 into register set (s + 1) % 2. The words of a
// step t are dequantised during the first three K groups of step t - 1 (words 0-1, 2 and 3 of a
// thread's four), their VALU work and LDS writes pinned between the MFMAs. The barrier waits for
// every load but the words last issued (`vmcnt(3)`), so those stay in flight for the next step as
// well; the dequantisation's own compiler-placed wait takes them.
//   issue_a(set, tile, ks): load the words of step (tile, ks) into set `set` (integral_constant)
//   commit_a(set, stageA, w0, w1): dequantise words [w0, w1) of set `set` into stageA
//   issue_b(tile, ks, stageB): B's direct loads of step (tile, ks)
// With an odd number nk of K steps a tile runs nk + 1, the last (ks == nk) staging zeros in both
// operands, so that the steps come in pairs; issue_a and issue_b see ks == nk there.
// ------------------------------------------------------------------------------------------
// Pins the order of one scheduling region of a 4-bit step: kMfma MFMAs, with kReads LDS reads
// spread over the first three quarters of them, one of kLoads vector-memory loads after each of
// the first kLoads MFMAs, kValu VALU instructions after every MFMA and kWrites LDS writes spread
// evenly (each after its share of the VALU work). The region ends with sched_barrier(0) at the
// caller, so that the dequantisation cannot gather in one block and loads keep their order across
// regions.
template <int kMfma, int kReads, int kLoads, int kValu, int kWrites>
__device__ __forceinline__ void sched_region() {
  constexpr int kSpan = kMfma * 3 / 4 > 0 ? kMfma * 3 / 4 : 1;
  static_assert(kLoads <= kMfma, "one load per MFMA");
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const int n = i < kSpan ? (i + 1) * kReads / kSpan - i * kReads / kSpan : 0;
    if (n == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (n == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (n == 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    if (i < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if (kValu > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    if (kWrites > 0 && (i + 1) % (kMfma / kWrites) == 0)
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  }
}

// The MFMAs of rows blocks MB0 and MB0 + 1 of one K group (half of mma_group).
template <class E, int MB0>
__device__ __forceinline__ void mma_half(f32x16 (&acc)[4][2], const typename E::Frag (&a)[4],
                                         const typename E::Frag (&b)[2],
                                         const typename E::Scales& sc) {
  E::template mma<MB0, 0>(acc[MB0][0], a[MB0], b[0], sc);
  E::template mma<MB0, 1>(acc[MB0][1], a[MB0], b[1], sc);
  E::template mma<MB0 + 1, 0>(acc[MB0 + 1][0], a[MB0 + 1], b[0], sc);
  E::template mma<MB0 + 1, 1>(acc[MB0 + 1][1], a[MB0 + 1], b[1], sc);
}

// The workgroup barrier of a 4-bit K-major step: this wave's LDS writes done, and every vector
// load except its last kLoadsA (the weight words just issued, which the next step's dequantisation
// waits for itself), so that the step's direct loads into the stage read next are done. In inline
// assembly: __syncthreads() would wait for every load.
template <int kLoadsA>
__device__ __forceinline__ void barrier_keep_words() {
  static_assert(kLoadsA == 3, "the wait count below");
  asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool kClear, int kLoadsA, class IssueA, class CommitA, class IssueB, class Epi>
__device__ __forceinline__ void gemm_run_q4k(const Smem& sm, int n_tiles, int nk, IssueA&& issue_a,
                                             CommitA&& commit_a, IssueB&& issue_b, Epi&& epi,
                                             f32x16 (&acc)[4][2]) {
  typedef EBf16 E;
  constexpr int kG = E::kGroups;
  static_assert(kG == 4, "the dequantisation of a step is split over the first three K groups");
  constexpr int kLoadsB = 4;   // DmaKS issues four direct loads per thread
  constexpr int kReads = 4 * reads_per_frag<E, true>() + 2 * reads_per_frag<E, true>();
  constexpr int kMfma = 8 * mfma_per_mma<E>();
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  // An odd nk gets one more K step per tile that stages zeros (see above), for an even total.
  const int nkp = nk + (nk & 1);
  const int total = n_tiles * nkp;
  if (total <= 0) return;
  const typename E::Scales sc{};
  const std::integral_constant<int, 0> set0{};
  const std::integral_constant<int, 1> set1{};
  typedef std::integral_constant<int, 0> W0;
  typedef std::integral_constant<int, 2> W2;
  typedef std::integral_constant<int, 3> W3;
  typedef std::integral_constant<int, 4> W4;
  StepPos cur{0, 0}, pa{0, 0}, pb{0, 0};
  issue_b(pb.tile, pb.ks, sm.b0);
  pb.next(nkp);
  issue_a(set0, pa.tile, pa.ks);   // step 0
  pa.next(nkp);
  issue_a(set1, pa.tile, pa.ks);   // step 1
  pa.next(nkp);
  commit_a(set0, sm.a0, W0{}, W4{});
  issue_a(set0, pa.tile, pa.ks);   // step 2
  pa.next(nkp);
  issue_b(pb.tile, pb.ks, sm.b1);  // step 1
  pb.next(nkp);
  vm_wait_seen();
  __syncthreads();
  FragSets<E> f;
  load_frags<E, true, true>(sm.a0, sm.b0, 0, wm, wn, l, f.a[0], f.b[0]);
  auto step = [&](auto parity, int s, char* __restrict__ ca, char* __restrict__ cb,
                  char* __restrict__ na, char* __restrict__ nb) {
    const std::integral_constant<int, 1 - decltype(parity)::value> next_set{};
    // Groups 0-2: step s + 1's words (set s + 1, loaded after step s - 2's barrier) into its
    // stage, words 0-1, 2 and 3.
    auto group = [&](auto kg_c, auto w0_c, auto w1_c) {
      constexpr int kg = decltype(kg_c)::value;
      constexpr int kWords = decltype(w1_c)::value - decltype(w0_c)::value;
      load_frags<E, true, true>(ca, cb, kg + 1, wm, wn, l, f.a[(kg + 1) & 1], f.b[(kg + 1) & 1]);
      mma_group<E>(acc, f.a[kg & 1], f.b[kg & 1], sc);
      commit_a(next_set, na, w0_c, w1_c);
      sched_region<kMfma, kReads, 0, (kWords * 30 + kMfma - 1) / kMfma, kWords>();
      __builtin_amdgcn_sched_barrier(0);
    };
    group(std::integral_constant<int, 0>{}, W0{}, W2{});
    group(std::integral_constant<int, 1>{}, W2{}, W3{});
    group(std::integral_constant<int, 2>{}, W3{}, W4{});
    const bool ends_tile = cur.ks == nkp - 1;
    barrier_keep_words<kLoadsA>();
    // Group 3: B's direct loads of step s + 2 with the first half of the MFMAs and the next
    // stage's first fragment reads, then (a region of its own, so that they follow the direct
    // loads and the next barrier can leave them in flight) step s + 3's words into the set
    // committed above with the second half.
    issue_b(pb.tile, pb.ks, cb);
    pb.next(nkp);
    load_frags<E, true, true>(na, nb, 0, wm, wn, l, f.a[0], f.b[0]);
    mma_half<E, 0>(acc, f.a[(kG - 1) & 1], f.b[(kG - 1) & 1], sc);
    sched_region<kMfma / 2, kReads, kLoadsB, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    issue_a(next_set, pa.tile, pa.ks);
    pa.next(nkp);
    mma_half<E, 2>(acc, f.a[(kG - 1) & 1], f.b[(kG - 1) & 1], sc);
    sched_region<kMfma / 2, 0, kLoadsA, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    if (ends_tile) {
      epi(cur.tile, acc);
      if (kClear) zero_acc(acc);
    }
    cur.next(nkp);
  };
  // An even number of steps, so that no path leads from the first step's loads back to the loop
  // header (the compiler would then wait there, on every iteration, for the words just issued).
  for (int it = 0; it < total; it += 2) {
    step(set0, it, sm.a0, sm.b0, sm.a1, sm.b1);
    step(set1, it + 1, sm.a1, sm.b1, sm.a0, sm.b0);
  }
  vm_wait_seen();   // the loads past the last step
}

// ------------------------------------------------------------------------------------------
// The 4-bit head's dh loop: one tile, A (coefficients) K-major by direct loads, B the 4-bit weights
// N-major (transposing fragment reads, so the barrier sits at the end of each step, as in
// gemm_step_end). Step s issues A's loads of step s + 1 and the words of step s + 2 (into register
// set s % 2, dequantised during step s - 1), then runs its four K groups, dequantising the words of
// step s + 1 (set (s + 1) % 2, complete since the previous barrier) one word per group between the
// MFMAs into step s + 1's stage, which no wave reads after that barrier.
//   issue_a(ks, stageA): A's direct loads of step ks;  issue_b(set, ks): the words of step ks;
//   commit_b(set, stageB, w0, w1): dequantise words [w0, w1) of `set` into stageB.
// An odd step count gets one more step that stages zeros (both operands; issue_a and issue_b see
// ks == nk there), so that steps come in pairs.
// ------------------------------------------------------------------------------------------
template <int kLoadsB, class IssueA, class IssueB, class CommitB>
__device__ __forceinline__ void gemm_run_q4n(const Smem& sm, int nk, IssueA&& issue_a,
                                             IssueB&& issue_b, CommitB&& commit_b,
                                             f32x16 (&acc)[4][2]) {
  typedef EBf16 E;
  constexpr int kG = E::kGroups;
  static_assert(kG == 4, "the dequantisation of a step is split over four K groups");
  constexpr int kLoadsA = 4;   // DmaKS issues four direct loads per thread
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int wm = w >> 2, wn = w & 3;
  const int total = nk + (nk & 1);
  if (total <= 0) return;
  const typename E::Scales sc{};
  const std::integral_constant<int, 0> set0{};
  const std::integral_constant<int, 1> set1{};
  typedef std::integral_constant<int, 0> W0;
  typedef std::integral_constant<int, 4> W4;
  issue_a(0, sm.a0);
  issue_b(set0, 0);
  issue_b(set1, 1);
  commit_b(set0, sm.b0, W0{}, W4{});
  vm_wait_seen();
  __syncthreads();
  auto step = [&](auto parity, int s, char* __restrict__ ca, char* __restrict__ cb,
                  char* __restrict__ na, char* __restrict__ nb) {
    const std::integral_constant<int, 1 - decltype(parity)::value> next_set{};
    issue_a(s + 1, na);
    issue_b(parity, s + 2);          // the set committed during the previous step
    FragSets<E> f;
    load_frags<E, true, false>(ca, cb, 0, wm, wn, l, f.a[0], f.b[0]);
    auto group = [&](auto kg_c) {
      constexpr int kg = decltype(kg_c)::value;
      if constexpr (kg + 1 < kG)
        load_frags<E, true, false>(ca, cb, kg + 1, wm, wn, l, f.a[(kg + 1) & 1], f.b[(kg + 1) & 1]);
      mma_group<E>(acc, f.a[kg & 1], f.b[kg & 1], sc);
      commit_b(next_set, nb, kg_c, std::integral_constant<int, kg + 1>{});
      sched_region<8 * mfma_per_mma<E>(),
                   (kg + 1 < kG) ? 4 * reads_per_frag<E, true>() + 2 * reads_per_frag<E, false>() : 0,
                   kg == 0 ? kLoadsA + kLoadsB : 0, (30 + 8 * mfma_per_mma<E>() - 1) / (8 * mfma_per_mma<E>()),
                   1>();
      __builtin_amdgcn_sched_barrier(0);
    };
    group(std::integral_constant<int, 0>{});
    group(std::integral_constant<int, 1>{});
    group(std::integral_constant<int, 2>{});
    group(std::integral_constant<int, 3>{});
    vm_wait_seen();
    __syncthreads();
  };
  // Steps in pairs: no path from the first step's loads back to the loop header.
  for (int it = 0; it < total; it += 2) {
    step(set0, it, sm.a0, sm.b0, sm.a1, sm.b1);
    step(set1, it + 1, sm.a1, sm.b1, sm.a0, sm.b0);
  }
  vm_wait_seen();
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on XCD b % 8), each with
// its own L2. xcd_remap(b, n) is a bijection of [0, n) under which every XCD processes one
// contiguous range of logical tiles, so the ~32 tiles an XCD runs at once share operand slices in
// its L2 instead of each slice being fetched into several L2s.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, i = b >> 3, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

// Position of accumulator element r of block (mb, nb) in the 256 x 256 tile.
__device__ __forceinline__ int acc_m(int wm, int mb, int r, int l) {
  return wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_n(int wn, int nb, int l) { return wn * 64 + nb * 32 + (l & 31); }

}  // namespace orpo
