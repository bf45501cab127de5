// gemm_mfma.hip - binary x ternary and ternary x ternary products on the
// matrix cores of gfx950, with {-1, 0, +1} operands encoded as FP4 (e2m1) and
// multiplied by v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales, fp32
// accumulation).
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: a binary/ternary MatMul for the
// linear and the attention operators, on bit-packed operands.  The product is
//   acc[m][n] = sum_k t[m][k] * s[n][k],   t in {-1,0,+1}, s in {-1,+1} (or t),
// rescaled by alpha_a[m] * alpha_b[n] in the fused epilogue.
//
// Exactness: -1, 0 and +1 are exact e2m1 values, every product is -1, 0 or +1,
// and every partial sum is an integer of magnitude <= K <= 65536 < 2^24, so
// the fp32 accumulation is exact in any order and converts to the int32 sum
// without rounding.
//
// Design (gfx950 first, not the page's CUDA kernel):
// * FP4 is the narrowest operand the matrix cores take: a 32x32x64 FP4 MFMA
//   does twice the k of the 32x32x32 int8 one in the same issue time, and a
//   4-bit element is cheap to build from the bit planes.
// * One wave owns a 128 x 128 output tile (4 x 4 MFMA tiles of 32 x 32, 256
//   fp32 accumulators per lane in AGPRs, one wave per SIMD).
// * The packed planes of each 256-k step (32 bytes per row and plane) are
//   copied global -> LDS with direct 16-byte DMA loads into a 3-deep ring per
//   wave; lane (r, g) reads its 16 bytes of each row (32-bit words w0..w3 of
//   half g) one step ahead and builds the MFMA operands in registers.
// * k order: the order of k inside an MFMA is free as long as A and B agree
//   (A nibble i of lane (r, g) meets B nibble i of lane (c, g)).  Slice e
//   (0..3) of a step puts into nibble j of operand word x the bit 4j + e of
//   source word wx.  Then an e2m1 nibble (bit 3 sign, bits 2..1 exponent,
//   +1 = 0x2, -1 = 0xA) is a shift and a mask away:
//     binary s  : ((w << (3 - e)) & 0x88888888) | 0x22222222
//     ternary t : q01 = bfi(0x33333333, m, s << 2), q23 = bfi(0x33333333, m >> 2, s)
//                 (mask and sign bits of k = 4j+e and 4j+e+1 side by side),
//                 slice 0: (q01 << 1) & 0xAAAAAAAA, 1: q01 & 0xAAAAAAAA,
//                 slice 2: (q23 << 1) & 0xAAAAAAAA, 3: q23 & 0xAAAAAAAA
//   (a zero mask bit with a stray sign bit gives -0, which adds nothing).
// * Software pipeline: the operands of slice e+1 are built while the 16 MFMAs
//   of slice e run, and the next step's words are read, re-laid and built into
//   slice 0 during slice 3, so the matrix cores never wait for a step boundary.
// * K is split over S waves of one block (S in {1, 2, 4}) when the grid would
//   otherwise leave SIMDs idle; the partial tiles are summed exactly in LDS.
//   Grids of unsplit tiles can instead pair a block's two waves on adjacent
//   column tiles that load their shared A panel once.
// * Tiles go to the XCDs in bands of 8 tile rows, so each XCD's L2 holds a
//   compact set of A and B panels; complete tiles store their output rows
//   through LDS, whole rows per 16-byte store.
#include <algorithm>
#include <vector>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int TILES = 4;  // 32-row MFMA tiles per wave along M and along N
constexpr int WAVE_TILE = 32 * TILES;
constexpr int kRing = 3;  // LDS stages per wave
constexpr int kFmtFp4 = 4;       // cbsz / blgp format code of e2m1
constexpr int kScaleOne = 127;   // E8M0 block scale 2^0

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y) {
  return (x & mask) | (y & ~mask);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS staging of one step (256 k = 32 bytes of each of 128 rows per plane).
// Plane order in a stage: A mask, A sign, B sign, [B mask].
// PAIR: two waves of a block on tiles (m, 2c) and (m, 2c + 1) share A; a slot
// holds A mask, A sign, B sign of wave 0 and of wave 1, [B mask of each], and
// each wave loads one A plane and its own B planes.
template <bool B_TERNARY, bool PAIR = false>
struct Stage {
  static constexpr int kPlane = WAVE_TILE * 32;
  static constexpr int kBPlanes = B_TERNARY ? 2 : 1;
  static constexpr int kPlanes = PAIR ? 2 + 2 * kBPlanes : 2 + kBPlanes;
  static constexpr int kBytes = kPlane * kPlanes;
  static constexpr int kLoads = 4 * (PAIR ? 1 + kBPlanes : kPlanes);  // DMA instructions per step and lane
};

// Copy 32 bytes (one 256-k step) of each of 128 rows of one plane into LDS
// with direct buffer->LDS 16-byte loads: lane i of instruction j moves half
// h = (i & 1) ^ ((i >> 4) & 1) of row 32j + i/2, and the hardware stores lane
// i's 16 bytes at dst + 16 i, so row rho lands at dst + 32 rho with its two
// halves swapped when bit 3 of rho is set.  Rows r and r + 8 of a 16-byte read
// (256 bytes apart) would share banks; the swap moves one of them to the other
// half (the bank-conflict counter of the q/k/v launch fell from 1.85 M to
// 0.43 M).  Loads go through a raw buffer
// descriptor of the tile's first row (base in SGPRs): the lane offset `off[j]`
// is the VGPR offset, the step's byte offset `soff` the scalar one, so no
// address arithmetic runs per load.  (Word 3 of the descriptor: 32-bit data
// format, the value the gfx9 raw-buffer convention uses; no range check is
// relied on, every offset stays inside the plane.)
//
// Lane offsets, computed once: off[j] = rho_j * row_bytes + h * 16 with
// rho_j = min(32j + lane/2, valid - 1) (rows past `valid` reuse the last valid
// row; their results are never stored).  The step that holds the row end
// (row_bytes % 32 != 0) uses offsets that include its byte offset, with every
// source kept inside the row:
// * a half that starts past the row end reads the row start instead;
// * a half that straddles the row end (row_bytes % 16 == 8) reads the 16 bytes
//   that end at the row end, i.e. the row's last 64-bit word lands in the
//   upper slot and the lower slot repeats the word before it.  B is staged the
//   same way, so the pairs still meet.
// Both kinds of stray A words are cleared in LDS before they are read
// (clear_tail).  This needs row_bytes >= 16 (K > 64), which the launcher
// guarantees.  A's 32-row blocks are also rotated by `rot` (LDS block t holds
// the tile's rows 32 ((t + rot) % 4) ..), so that with split K the rows a wave
// keeps are always its accumulators acc[0 .. 4/S).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base) {
  // The base goes through readfirstlane: the descriptor must live in SGPRs, and
  // the compiler does not always prove the tile origin wave-uniform.
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, 0x7FFFFFFF, 0x00020000);
}

__device__ __forceinline__ void dma_plane(__amdgpu_buffer_rsrc_t rsrc, const uint32_t (&off)[4],
                                          uint32_t soff, uint8_t* dst) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + j * 1024), 16, off[j], soff,
                                             0, 0);
}

// s_waitcnt immediate for "vmcnt <= n" (expcnt and lgkmcnt at their no-wait
// maxima); vmcnt is split over bits 3:0 and 15:14.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

typedef uint32_t Words[TILES][4];  // 32-bit words 4g..4g+3 of rows 32t + r

// LDS address of half g of staged row rho (the DMA's half swap).
__device__ __forceinline__ int stage_off(int rho, int g) {
  return rho * 32 + 16 * (g ^ ((rho >> 3) & 1));
}

// Lane (r, g) reads its 16 bytes of row 32t + r of one staged plane.
__device__ __forceinline__ void read_words(Words& w, const uint8_t* plane, int r, int g) {
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(plane + stage_off(32 * t + r, g));
#pragma unroll
    for (int x = 0; x < 4; ++x) w[t][x] = v[x];
  }
}

// In the step that holds the row end, zero the A mask words of lane (r, g)
// that lie past the row end or repeat the word before a straddling window, so
// that they contribute nothing (a zero mask bit makes the A element +-0).
// Each lane clears only the bytes it reads itself.
__device__ __forceinline__ void clear_tail(uint8_t* stage, int r, int g, int st, int words,
                                           bool straddle) {
  const int kw = st * 4 + 2 * g;  // 64-bit word index of slot 0
  const bool sh = straddle && kw == words - 1;
  const bool keep0 = kw < words && !sh;
  const bool keep1 = kw + 1 < words || sh;
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    uint64_t* w = reinterpret_cast<uint64_t*>(stage + stage_off(32 * t + r, g));
    if (!keep0) w[0] = 0;
    if (!keep1) w[1] = 0;
  }
}

// Ternary words with the (mask, sign) bits of k = 4j+e and 4j+e+1 side by
// side: q01 for slices 0, 1 and q23 for slices 2, 3.
__device__ __forceinline__ void prep_q01(const Words& m, const Words& s, Words& q) {
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x) q[t][x] = bfi(0x33333333u, m[t][x], s[t][x] << 2);
}
__device__ __forceinline__ void prep_q23(const Words& m, const Words& s, Words& q) {
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x) q[t][x] = bfi(0x33333333u, m[t][x] >> 2, s[t][x]);
}

// e2m1 operands of slice e: ternary from q01 (e = 0, 1) or q23 (e = 2, 3).
__device__ __forceinline__ void ternary_slice(const Words& q, int e, v4i (&o)[TILES]) {
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x) o[t][x] = (int)((e & 1 ? q[t][x] : q[t][x] << 1) & 0xAAAAAAAAu);
}

// Binary operand of slice e: the sign bit moved to nibble bit 3 and merged with
// the +1 pattern 0x22222222 by one v_bitop3_b32 (table 0xE2: S1 ? S0 : S2 with
// the index S0*4 + S1*2 + S2).
__device__ __forceinline__ void binary_slice(const Words& w, int e, v4i (&o)[TILES]) {
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x)
      o[t][x] = (int)__builtin_amdgcn_bitop3_b32(w[t][x] << (3 - e), 0x88888888u, 0x22222222u,
                                                 0xE2);
}

__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, v16f c) {
  const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
  const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 0, kScaleOne,
                                                          0, kScaleOne);
}

// LDS of the cross-wave reduction: every wave's partial sums of one owner's
// rows, 64 KiB in all (within the rings whenever S > 1).
constexpr size_t kXchgBytes = (size_t)TILES * TILES * 16 * kWave * 4;

// Two fp32 values as a bf16 pair (low half first), each rounded to nearest
// even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Store row block i (32 rows x 32 NJ columns) of a complete tile from the
// lanes' output words o[j][qh][..] (row r, columns 32 j + 8 qh + 4 g + 0..3;
// ES = 4: one fp32 or int32 per word, ES = 2: bf16 pairs in words 0 and 1).
// In that layout a store instruction covers 32 rows x 4 elements, one L2
// request per row, so the block goes through LDS (stg: the wave's own, free
// staging area) row-major, and each 16-byte store instruction then writes whole
// rows: 64 lanes x 16 bytes over 64 lanes / (2 NJ ES) rows, a quarter to an
// eighth of the requests.
template <int NJ, int ES>
__device__ __forceinline__ void store_row_block(const uint32_t (&o)[TILES][4][4], uint8_t* stg,
                                                int r, int g, int lane,
                                                __amdgpu_buffer_rsrc_t yrs, uint32_t ldb, int i) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  constexpr int RB = 32 * NJ * ES;  // bytes of one row of the block
  constexpr int PITCH = RB + 16;    // staged row pitch (rows on different banks)
  constexpr int LPR = RB / 16;      // lanes per row in a 16-byte read
  constexpr int RPI = kWave / LPR;  // rows per store instruction
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int qh = 0; qh < 4; ++qh) {
      const uint32_t(&w)[4] = o[j][qh];
      uint8_t* dst = stg + r * PITCH + (32 * j + 8 * qh + 4 * g) * ES;
      if constexpr (ES == 4)
        *reinterpret_cast<v4u*>(dst) = v4u{w[0], w[1], w[2], w[3]};
      else
        *reinterpret_cast<v2u*>(dst) = v2u{w[0], w[1]};
    }
  // other lanes read what this lane wrote: complete the writes first
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  const int soff = (int)__builtin_amdgcn_readfirstlane(32 * i * ldb);
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / LPR;
    const int cb = (lane % LPR) * 16;
    const v4u d = *reinterpret_cast<const v4u*>(stg + rr * PITCH + cb);
    __builtin_amdgcn_raw_buffer_store_b128(d, yrs, (int)(rr * ldb + cb), soff, 0);
  }
  // and the reads before the next row block overwrites the stage
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// RES: B holds two binary planes per weight row, interleaved in groups of 32
// rows (plane 1 of weight rows 32p..32p+31, then plane 2 of the same rows), so
// MFMA column tiles 2jj and 2jj + 1 of a wave tile carry the two accumulators of
// the same 32 outputs in the same lanes, and the epilogue writes
// y = acc1 * (alpha_a * alpha1) + acc2 * (alpha_a * alpha2) to N / 2 columns.
constexpr int kBand = 8;  // tile rows per band of the tile order

// One block's tile: the whole kernel but for the block's index `vblk` among the
// `vnblk` blocks of its part of the launch (the launch, or one part of a
// two-part launch).
template <bool B_TERNARY, int OUT, int S, bool RES = false, bool PAIR = false>
__device__ __forceinline__ void gemm_tile(
    const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
    const float* __restrict__ a_alpha, int64_t a_batch_rows, const uint8_t* __restrict__ b_mask,
    const uint8_t* __restrict__ b_sign, const float* __restrict__ b_alpha, int64_t b_batch_rows,
    int64_t M, int64_t N, int64_t row_bytes, int tiles_m, int tiles_n, void* __restrict__ Y,
    int64_t ldy, int64_t y_batch_stride, int tile0, int vblk, int vnblk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = __lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = lane & 31;
  const int g = lane >> 5;

  // The part covers tiles tile0 .. tile0 + vnblk - 1 of the tile order
  // below.  Blocks are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of that order, whose tiles then share A and B panels in the
  // XCD's L2 (a part that starts at a multiple of 8 blocks keeps the deal).  Order: bands of kBand tile rows, column by column within a band,
  // so a run of r tiles spans about kBand rows and r / kBand columns (LLaMA-7B
  // gate and up as separate products, 172 tiles per XCD: 1 MB of A and 1.4 MB of
  // B panels, against 0.25 MB and all 5.6 MB of B for row-major runs).
  const int nblk = vnblk;
  int lin = vblk;
  if ((nblk & 7) == 0) lin = (vblk & 7) * (nblk >> 3) + (vblk >> 3);
  lin += tile0;
  // PAIR: the order runs over column pairs; wave w takes column 2c + w (a
  // missing last column repeats column tiles_n - 1 and stores nothing)
  const int tn_order = PAIR ? (tiles_n + 1) / 2 : tiles_n;
  const int band = lin / (kBand * tn_order);
  const int band_rows = min(kBand, tiles_m - band * kBand);
  const int in_band = lin - band * kBand * tn_order;
  const int tile_c = in_band / band_rows;
  const int tile_m = band * kBand + (in_band - tile_c * band_rows);
  const bool store_ok = !PAIR || 2 * tile_c + wid < tiles_n;
  const int tile_n = PAIR ? min(2 * tile_c + wid, tiles_n - 1) : tile_c;
  const int64_t b = blockIdx.z;
  const int64_t m0 = (int64_t)tile_m * WAVE_TILE;
  const int64_t n0 = (int64_t)tile_n * WAVE_TILE;
  const int m_valid = (int)(M - m0 < WAVE_TILE ? M - m0 : WAVE_TILE);
  const int n_valid = (int)(N - n0 < WAVE_TILE ? N - n0 : WAVE_TILE);

  const int64_t a_row0 = b * a_batch_rows + m0;
  const int64_t b_row0 = b * b_batch_rows + n0;
  const uint8_t* am = a_mask + a_row0 * row_bytes;
  const uint8_t* as = a_sign + a_row0 * row_bytes;
  const uint8_t* bm = B_TERNARY ? b_mask + b_row0 * row_bytes : nullptr;
  const uint8_t* bs = b_sign + b_row0 * row_bytes;

  const int64_t words = row_bytes / 8;          // 64-bit words per row
  const int64_t steps = (words + 3) / 4;        // 4 words (256 k) per step
  static_assert(!PAIR || S == 1, "paired waves each run the whole K range");
  const int64_t st0 = PAIR ? 0 : steps * wid / S;
  const int64_t st1 = PAIR ? steps : steps * (wid + 1) / S;
  constexpr int TPW = TILES / S;  // 32-row blocks of the tile each wave finally owns
  const int rot = PAIR ? 0 : wid * TPW;  // acc[t] accumulates the tile's row block (t + rot) % 4

  // The tile's scales: wave 0 (PAIR: each wave, for its own columns; both store
  // the same A scales) loads them first thing, the first DMAs go out behind
  // them, and the wait for the first step (which completes them too) precedes
  // their store to LDS, so their latency hides under the DMA's.
  __shared__ float s_alpha_a[WAVE_TILE], s_alpha_b[PAIR ? 2 : 1][WAVE_TILE];
  const int sw = PAIR ? wid : 0;
  float ra[WAVE_TILE / kWave], rbv[WAVE_TILE / kWave];
  const bool scale_wave = OUT != (int)Elt::I32 && (PAIR || wid == 0);
  if (scale_wave) {
#pragma unroll
    for (int h = 0; h < WAVE_TILE / kWave; ++h) {
      const int i = h * kWave + lane;
      ra[h] = i < m_valid ? a_alpha[b * a_batch_rows + m0 + i] : 0.0f;
      rbv[h] = i < n_valid ? b_alpha[b * b_batch_rows + n0 + i] : 0.0f;
    }
  }
  auto store_scales = [&]() {
    if (scale_wave) {
#pragma unroll
      for (int h = 0; h < WAVE_TILE / kWave; ++h) {
        s_alpha_a[h * kWave + lane] = ra[h];
        s_alpha_b[sw][h * kWave + lane] = rbv[h];
      }
    }
  };
  v16f acc[TILES][TILES];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int j = 0; j < TILES; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  constexpr int SB = Stage<B_TERNARY, PAIR>::kBytes;
  constexpr int P = Stage<B_TERNARY, PAIR>::kPlane;
  constexpr int L = Stage<B_TERNARY, PAIR>::kLoads;
  uint8_t* ring = PAIR ? smem : smem + (size_t)wid * kRing * SB;
  // plane offsets in a slot: A mask 0, A sign P, then this wave's B planes
  const int bs_off = PAIR ? (2 + wid) * P : 2 * P;
  const int bm_off = PAIR ? (4 + wid) * P : 3 * P;
  const uint32_t rb = (uint32_t)row_bytes;
  const bool straddle = (rb & 15u) == 8u;
  if (st0 < st1) {
    const int w32 = (int)words, s0i = (int)st0, s1i = (int)st1, last = s1i - 1;
    // DMA lane offsets: full-step form (offa/offb, plus the step's byte offset
    // as the scalar offset) until the step that holds the row end, whose own
    // offsets (offa_t/offb_t) replace them from then on.
    const int tail_st = (rb & 31u) ? (int)steps - 1 : 0x7FFFFFFF;
    uint32_t offa[4], offb[4], offa_t[4], offb_t[4];
    {
      const uint32_t half = (uint32_t)((lane & 1) ^ ((lane >> 4) & 1)) * 16;
      uint32_t ot = (uint32_t)(steps - 1) * 32 + half;
      if (ot + 16 > rb) ot = ot < rb ? rb - 16 : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t ra_ = (uint32_t)min(32 * ((j + rot) & 3) + (lane >> 1), m_valid - 1) * rb;
        const uint32_t rb_ = (uint32_t)min(32 * j + (lane >> 1), n_valid - 1) * rb;
        offa[j] = ra_ + half;
        offb[j] = rb_ + half;
        offa_t[j] = ra_ + ot;
        offb_t[j] = rb_ + ot;
      }
    }
    // Descriptors stay plain locals (inside an aggregate they can land in VGPRs).
    const __amdgpu_buffer_rsrc_t ras = uniform_rsrc(as), rbs = uniform_rsrc(bs);
    const __amdgpu_buffer_rsrc_t rbm = B_TERNARY ? uniform_rsrc(bm) : rbs;
    // PAIR: wave 0 loads the shared A mask plane, wave 1 the A sign plane
    const __amdgpu_buffer_rsrc_t rao = uniform_rsrc(PAIR && wid ? as : am);
    const int ao_off = PAIR ? wid * P : 0;
    // PAIR: the other wave's DMAs of a step (and its reads of the slot about to
    // be refilled) are done once both waves have passed their own wait
    auto pair_sync = [&]() {
      if constexpr (PAIR) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      }
    };
    // Ring of 3 slots: step s0i + i lives in slot i % 3.  Steps past the wave's
    // range reload its last step (never used), which keeps the wait counts
    // uniform.  step_soff() picks the step (clamped) and returns its scalar
    // offset, switching to the row-end offsets when it gets there.
    auto step_soff = [&](int st) -> uint32_t {
      const int sd = min(st, last);
      if (sd == tail_st) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          offa[j] = offa_t[j];
          offb[j] = offb_t[j];
        }
        return 0u;
      }
      return (uint32_t)sd * 32;
    };
    auto dma = [&](int st, uint8_t* slot) {  // all planes of one step
      const uint32_t so = step_soff(st);
      dma_plane(rao, offa, so, slot + ao_off);
      if constexpr (!PAIR) dma_plane(ras, offa, so, slot + P);
      dma_plane(rbs, offb, so, slot + bs_off);
      if constexpr (B_TERNARY) dma_plane(rbm, offb, so, slot + bm_off);
    };
    uint8_t* slot0 = ring;           // step st
    uint8_t* slot1 = ring + SB;      // step st + 1
    uint8_t* slot2 = ring + 2 * SB;  // step st + 2

    // Registers, for the step st being multiplied:
    //   qa01/qa23 (and qb01/qb23): its prepared ternary words;  wb: its binary
    //   B words;  na_m/na_s (nb_m/nb_s): raw words of a later step;
    //   oa/ob: operands of the slice in flight and of the next one.
    Words qa01, qa23, qb01, qb23, wb, na_m, na_s, nb_m, nb_s;
    v4i oa[2][TILES], ob[2][TILES];

    auto ready = [&](int st, uint8_t* slot) {  // stray A words of the row-end step
      if (st * 32 + 32 > (int)rb) clear_tail(slot, r, g, st, w32, straddle);
    };
    dma(s0i, slot0);
    dma(s0i + 1, slot1);
    dma(s0i + 2, slot2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));  // step st0 (and the scales) landed
    pair_sync();
    store_scales();
    ready(s0i, slot0);
    read_words(na_m, slot0, r, g);
    read_words(na_s, slot0 + P, r, g);
    if constexpr (B_TERNARY) {
      read_words(nb_s, slot0 + bs_off, r, g);
      read_words(nb_m, slot0 + bm_off, r, g);
      prep_q01(nb_m, nb_s, qb01);
      prep_q23(nb_m, nb_s, qb23);
      ternary_slice(qb01, 0, ob[0]);
    } else {
      read_words(wb, slot0 + bs_off, r, g);
      binary_slice(wb, 0, ob[0]);
    }
    prep_q01(na_m, na_s, qa01);
    prep_q23(na_m, na_s, qa23);
    ternary_slice(qa01, 0, oa[0]);

#define BWTA_MFMA_SLICE(C)                                                              \
  _Pragma("unroll") for (int i = 0; i < TILES; ++i)                                    \
  _Pragma("unroll") for (int j = 0; j < TILES; ++j)                                    \
      acc[i][j] = mfma_fp4(ob[C][j], oa[C][i], acc[i][j])
#define BWTA_REGION_END()                                                               \
  do {                                                                                  \
    _Pragma("unroll") for (int k = 0; k < TILES * TILES; ++k) {                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* 1 MFMA */                   \
      if (k % 4 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* 1 DMA */    \
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0); /* up to 6 VALU */             \
    }                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)

    // Per step st: at the top, wait for step st + 1 (st + 2 may still be in
    // flight), clear its stray words if it holds the row end, and start reading
    // step st + 1's A words.  Then four regions, one per slice, each running its
    // 16 MFMAs with the VALU work below spread between them, and each refilling
    // one plane of the slot of step st (all in registers by now) with step
    // st + 3:
    //   A: build slice 1;  prepare q01 of step st + 1 (q01 of st is done)
    //   B: build slice 2
    //   C: build slice 3;  re-read step st + 1's A words, prepare its q23;
    //      read its binary B words
    //   D: build slice 0 of step st + 1
    for (int st = s0i; st < s1i; ++st) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(L));
      pair_sync();
      ready(st + 1, slot1);
      const uint32_t so = step_soff(st + 3);
      read_words(na_m, slot1, r, g);
      read_words(na_s, slot1 + P, r, g);
      if constexpr (B_TERNARY) {
        read_words(nb_s, slot1 + bs_off, r, g);
        read_words(nb_m, slot1 + bm_off, r, g);
      }
      __builtin_amdgcn_sched_barrier(0);
      // A
      ternary_slice(qa01, 1, oa[1]);
      if constexpr (B_TERNARY)
        ternary_slice(qb01, 1, ob[1]);
      else
        binary_slice(wb, 1, ob[1]);
      prep_q01(na_m, na_s, qa01);
      if constexpr (B_TERNARY) prep_q01(nb_m, nb_s, qb01);
      dma_plane(rao, offa, so, slot0 + ao_off);  // step st + 3 into the slot of step st
      BWTA_MFMA_SLICE(0);
      BWTA_REGION_END();
      // B
      ternary_slice(qa23, 2, oa[0]);
      if constexpr (B_TERNARY)
        ternary_slice(qb23, 2, ob[0]);
      else
        binary_slice(wb, 2, ob[0]);
      if constexpr (!PAIR) dma_plane(ras, offa, so, slot0 + P);
      BWTA_MFMA_SLICE(1);
      BWTA_REGION_END();
      // C
      read_words(na_m, slot1, r, g);
      read_words(na_s, slot1 + P, r, g);
      if constexpr (B_TERNARY) {
        read_words(nb_s, slot1 + bs_off, r, g);
        read_words(nb_m, slot1 + bm_off, r, g);
      }
      ternary_slice(qa23, 3, oa[1]);
      if constexpr (B_TERNARY)
        ternary_slice(qb23, 3, ob[1]);
      else
        binary_slice(wb, 3, ob[1]);
      prep_q23(na_m, na_s, qa23);
      if constexpr (B_TERNARY)
        prep_q23(nb_m, nb_s, qb23);
      else
        read_words(wb, slot1 + bs_off, r, g);
      dma_plane(rbs, offb, so, slot0 + bs_off);
      BWTA_MFMA_SLICE(0);
      BWTA_REGION_END();
      // D
      ternary_slice(qa01, 0, oa[0]);
      if constexpr (B_TERNARY)
        ternary_slice(qb01, 0, ob[0]);
      else
        binary_slice(wb, 0, ob[0]);
      if constexpr (B_TERNARY) dma_plane(rbm, offb, so, slot0 + bm_off);
      BWTA_MFMA_SLICE(1);
      BWTA_REGION_END();
      uint8_t* const done = slot0;
      slot0 = slot1;
      slot1 = slot2;
      slot2 = done;
    }
#undef BWTA_MFMA_SLICE
#undef BWTA_REGION_END
  } else {
    store_scales();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may land in LDS from here on

  // Accumulator layout: acc[t][j] = B_j x A_i^T with i = (t + rot) % 4, i.e. the
  // MFMA's rows run over the output columns.  Register q of lane (r, g) holds
  // output element
  //   row 32i + r,  column 32j + 8 (q / 4) + 4g + q % 4,
  // so each lane owns runs of 4 consecutive columns.  The fp32 sums are exact
  // integers.
  //
  // Cross-wave reduction (S > 1): wave w owns the row blocks it holds in
  // acc[0 .. TPW) (blocks rot .. rot + TPW - 1) and, in round k, hands
  // acc[k TPW .. (k+1) TPW) - the blocks of wave (w + k) % S - to that wave
  // through LDS, in a lane-major layout (each lane moves its own registers, 16
  // bytes at a time), while adding wave (w - k) % S's share of its own blocks.
  // fp32 adds of integers below 2^24 are exact.
  if constexpr (S > 1) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    v4f* xbuf = reinterpret_cast<v4f*>(smem);
    constexpr int region = TPW * TILES * 4 * kWave;  // float4s per wave
    __syncthreads();  // every wave is done with its ring
#pragma unroll
    for (int k = 1; k < S; ++k) {
      const int from = (wid - k) & (S - 1);
#pragma unroll
      for (int ii = 0; ii < TPW; ++ii)
#pragma unroll
        for (int j = 0; j < TILES; ++j) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const v16f& a = acc[k * TPW + ii][j];
            const v4f v = {a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
            xbuf[wid * region + ((ii * TILES + j) * 4 + c) * kWave + lane] = v;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      __syncthreads();
#pragma unroll
      for (int ii = 0; ii < TPW; ++ii)
#pragma unroll
        for (int j = 0; j < TILES; ++j) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const v4f v = xbuf[from * region + ((ii * TILES + j) * 4 + c) * kWave + lane];
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[ii][j][4 * c + u] += v[u];
          }
          __builtin_amdgcn_sched_barrier(0);  // one 32x32 tile at a time: few live VGPRs
        }
      __syncthreads();
    }
  }

  // The tile's scales were stored to LDS by other lanes (of wave 0): order those
  // stores before the reads below (the compiler orders memory per lane only).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  if (!store_ok) return;  // PAIR: the repeated last column
  // Staging area of this wave's row blocks: its own ring, or (PAIR, one ring
  // per block) its half of the block's ring, free once both waves are here.
  uint8_t* const stg = PAIR ? smem + (size_t)wid * (WAVE_TILE * 4 + 16) * 32
                            : smem + (size_t)wid * kRing * Stage<B_TERNARY>::kBytes;

  // Epilogue straight from the registers of the owned tile rows: y = acc *
  // (alpha_a[row] * alpha_b[col]) in fp32 (the product of the scales first),
  // bf16 rounded to nearest even (v_cvt_pk_bf16_f32), or the int32 sum itself.
  // Complete tiles store row blocks through LDS (store_row_block: whole rows per
  // 16-byte store, through a buffer descriptor of the tile origin); edge tiles
  // store a lane's elements one by one with every element checked.
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  char* ytile = static_cast<char*>(Y) + (b * y_batch_stride + m0 * ldy + (RES ? n0 / 2 : n0)) * ES;
  // The column scales of this lane's 64 columns, read once.
  float ab[TILES][4][4];
#pragma unroll
  for (int j = 0; j < TILES; ++j)
#pragma unroll
    for (int qh = 0; qh < 4; ++qh) {
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if constexpr (OUT != (int)Elt::I32)
        v = *reinterpret_cast<const float4*>(&s_alpha_b[sw][32 * j + 8 * qh + 4 * g]);
      ab[j][qh][0] = v.x;
      ab[j][qh][1] = v.y;
      ab[j][qh][2] = v.z;
      ab[j][qh][3] = v.w;
    }
  // The staged stores write 16 bytes at a time: they need a 16-byte aligned tile
  // origin and row pitch (the C interface asks only for element alignment).
  const bool full = m_valid == WAVE_TILE && n_valid == WAVE_TILE &&
                    (int64_t)WAVE_TILE * ldy * ES < (int64_t)0x7FFFFFFF &&
                    ((ldy * ES) & 15) == 0 && (reinterpret_cast<uintptr_t>(ytile) & 15) == 0;
  const __amdgpu_buffer_rsrc_t yrs = uniform_rsrc(ytile);
  const uint32_t ldb = (uint32_t)(ldy * ES);
  if constexpr (RES) {
    static_assert(OUT != (int)Elt::I32, "two-plane products are scaled");

    // n_valid is a multiple of 64 (N / 2 a multiple of 32): whole output tiles.
    // The scales come straight from global memory (L2 hits: wave 0 read them).
    float ab2[TILES][4][4];
#pragma unroll
    for (int j = 0; j < TILES; ++j)
#pragma unroll
      for (int qh = 0; qh < 4; ++qh)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int col = 32 * j + 8 * qh + 4 * g + u;
          ab2[j][qh][u] = col < n_valid ? b_alpha[b * b_batch_rows + n0 + col] : 0.0f;
        }
#pragma unroll
    for (int ii = 0; ii < TPW; ++ii) {
      const int i = (ii + rot) & 3;
      const int row = 32 * i + r;
      const float aa = row < m_valid ? a_alpha[b * a_batch_rows + m0 + row] : 0.0f;
      uint32_t o[TILES][4][4];  // the first TILES / 2 column blocks are used
#pragma unroll
      for (int jj = 0; jj < TILES / 2; ++jj)
#pragma unroll
        for (int qh = 0; qh < 4; ++qh) {
          float y[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float y1 = acc[ii][2 * jj][4 * qh + u] * (aa * ab2[2 * jj][qh][u]);
            const float y2 = acc[ii][2 * jj + 1][4 * qh + u] * (aa * ab2[2 * jj + 1][qh][u]);
            y[u] = y1 + y2;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if constexpr (OUT == (int)Elt::F32)
              o[jj][qh][u] = __float_as_uint(y[u]);
            else if (u < 2)
              o[jj][qh][u] = pack_bf16x2(y[2 * u], y[2 * u + 1]);
          }
        }
      if (full) {
        store_row_block<TILES / 2, ES>(o, stg, r, g, lane, yrs, ldb, i);
      } else if (row < m_valid) {
#pragma unroll
        for (int jj = 0; jj < TILES / 2; ++jj)
#pragma unroll
          for (int qh = 0; qh < 4; ++qh)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int col = 32 * jj + 8 * qh + 4 * g + u;
              if (col < n_valid / 2) {
                char* yp = ytile + ((int64_t)row * ldy + col) * ES;
                if constexpr (ES == 4)
                  *reinterpret_cast<uint32_t*>(yp) = o[jj][qh][u];
                else
                  *reinterpret_cast<uint16_t*>(yp) = (uint16_t)(o[jj][qh][u >> 1] >> (16 * (u & 1)));
              }
            }
      }
    }
    return;
  }
  // Per owned row block: every accumulator is read once into the output words
  // (4 consecutive columns per (j, qh)), then stored - wide when the tile is
  // complete, element by element with bounds checks otherwise.
#pragma unroll
  for (int ii = 0; ii < TPW; ++ii) {
    const int i = (ii + rot) & 3;  // tile row block of acc[ii]
    const int row = 32 * i + r;
    const float aa = OUT != (int)Elt::I32 ? s_alpha_a[row] : 0.0f;
    uint32_t o[TILES][4][4];
#pragma unroll
    for (int j = 0; j < TILES; ++j)
#pragma unroll
      for (int qh = 0; qh < 4; ++qh) {
        if constexpr (OUT == (int)Elt::BF16) {
          float y[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) y[u] = acc[ii][j][4 * qh + u] * (aa * ab[j][qh][u]);
          o[j][qh][0] = pack_bf16x2(y[0], y[1]);
          o[j][qh][1] = pack_bf16x2(y[2], y[3]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float a = acc[ii][j][4 * qh + u];
            if constexpr (OUT == (int)Elt::I32)
              o[j][qh][u] = (uint32_t)(int)a;
            else
              o[j][qh][u] = __float_as_uint(a * (aa * ab[j][qh][u]));
          }
        }
      }
    if (full) {
      store_row_block<TILES, ES>(o, stg, r, g, lane, yrs, ldb, i);
    } else if (row < m_valid) {
#pragma unroll
      for (int j = 0; j < TILES; ++j)
#pragma unroll
        for (int qh = 0; qh < 4; ++qh)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int col = 32 * j + 8 * qh + 4 * g + u;
            if (col < n_valid) {
              char* yp = ytile + ((int64_t)row * ldy + col) * ES;
              if constexpr (ES == 4)
                *reinterpret_cast<uint32_t*>(yp) = o[j][qh][u];
              else
                *reinterpret_cast<uint16_t*>(yp) = (uint16_t)(o[j][qh][u >> 1] >> (16 * (u & 1)));
            }
          }
    }
  }
}

template <bool B_TERNARY, int OUT, int S, bool RES = false, bool PAIR = false>
__global__ void __launch_bounds__((PAIR ? 2 : S) * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_mfma_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                 const float* __restrict__ a_alpha, int64_t a_batch_rows,
                 const uint8_t* __restrict__ b_mask, const uint8_t* __restrict__ b_sign,
                 const float* __restrict__ b_alpha, int64_t b_batch_rows, int64_t M, int64_t N,
                 int64_t row_bytes, int tiles_m, int tiles_n, void* __restrict__ Y, int64_t ldy,
                 int64_t y_batch_stride, int tile0) {
  gemm_tile<B_TERNARY, OUT, S, RES, PAIR>(a_mask, a_sign, a_alpha, a_batch_rows, b_mask, b_sign,
                                          b_alpha, b_batch_rows, M, N, row_bytes, tiles_m, tiles_n,
                                          Y, ldy, y_batch_stride, tile0, (int)blockIdx.x,
                                          (int)gridDim.x);
}

// Two parts in one launch of two-wave blocks: blocks [0, npair) run paired waves
// over the first npair column pairs of the pair order (2 npair whole tiles),
// the rest split K in two over the single-tile order from tile 2 npair on (the
// host checks that the two orders cover the same first 2 npair tiles).  The
// second part's blocks start as the first part's retire, under their output
// stores, with no launch gap between the parts.
template <bool B_TERNARY, int OUT, bool RES = false>
__global__ void __launch_bounds__(2 * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_mfma_two_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                     const float* __restrict__ a_alpha, const uint8_t* __restrict__ b_mask,
                     const uint8_t* __restrict__ b_sign, const float* __restrict__ b_alpha,
                     int64_t M, int64_t N, int64_t row_bytes, int tiles_m, int tiles_n,
                     void* __restrict__ Y, int64_t ldy, int npair) {
  if ((int)blockIdx.x < npair)
    gemm_tile<B_TERNARY, OUT, 1, RES, true>(a_mask, a_sign, a_alpha, 0, b_mask, b_sign, b_alpha, 0,
                                            M, N, row_bytes, tiles_m, tiles_n, Y, ldy, 0, 0,
                                            (int)blockIdx.x, npair);
  else
    gemm_tile<B_TERNARY, OUT, 2, RES, false>(a_mask, a_sign, a_alpha, 0, b_mask, b_sign, b_alpha,
                                             0, M, N, row_bytes, tiles_m, tiles_n, Y, ldy, 0,
                                             2 * npair, (int)blockIdx.x - npair,
                                             (int)gridDim.x - npair);
}

// Split K over S waves when that fills more SIMDs: minimise rounds(S) / S, where a
// round is one wave on each of the 1024 SIMDs; no more waves than 256-k steps
// (BERT's 768 x 768 product, 3 steps on 192 tiles, takes S = 2: 384 waves of one
// or two steps instead of 192 waves of three).
int choose_split(int64_t tiles, int64_t steps) {
  const int64_t simds = 1024;
  int best = 1;
  double best_cost = 1e30;
  for (int S = 1; S <= 4; S *= 2) {
    if (S > 1 && steps < S) break;
    const double rounds = (double)((tiles * S + simds - 1) / simds);
    const double cost = rounds / S;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// tiles: blocks of the launch (PAIR: column pairs, two waves each).
template <bool B_TERNARY, int OUT, int S, bool RES = false, bool PAIR = false>
hipError_t launch_k(const GemmArgs& g, int64_t row_bytes, int64_t tm, int64_t tn, int64_t tile0,
                    int64_t tiles, hipStream_t stream) {
  size_t lds = (size_t)(PAIR ? 1 : S) * kRing * Stage<B_TERNARY, PAIR>::kBytes;
  if (S > 1 && lds < kXchgBytes) lds = kXchgBytes;
  auto kfn = gemm_mfma_kernel<B_TERNARY, OUT, S, RES, PAIR>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3((unsigned)tiles, 1, (unsigned)g.batch),
                     dim3((PAIR ? 2 : S) * kWave), lds,
                     stream, g.a_mask, g.a_sign, g.a_alpha, g.a_batch_rows, g.b_mask, g.b_sign,
                     g.b_alpha, g.b_batch_rows, g.M, g.N, row_bytes, (int)tm, (int)tn, g.Y, g.ldy,
                     g.y_batch_stride, (int)tile0);
  return hipGetLastError();
}

// Tile (row, column) of entry `lin` of the tile order (pair order: column pairs),
// as the kernel computes it.
void order_tile(int64_t lin, int64_t tm, int64_t tn, bool pair, int w, int64_t& r, int64_t& c) {
  const int64_t tn_order = pair ? (tn + 1) / 2 : tn;
  const int64_t band = lin / (kBand * tn_order);
  const int64_t band_rows = std::min<int64_t>(kBand, tm - band * kBand);
  const int64_t in_band = lin - band * kBand * tn_order;
  const int64_t tc = in_band / band_rows;
  r = band * kBand + (in_band - tc * band_rows);
  c = pair ? 2 * tc + w : tc;
}

// Whether the first npair entries of the pair order cover exactly the first
// 2 npair tiles of the single-tile order (then one two-part launch can run them).
bool pair_prefix_matches(int64_t tm, int64_t tn, int64_t npair) {
  if (tn % 2 != 0 || 2 * npair > tm * tn) return false;
  std::vector<char> seen((size_t)(tm * tn), 0);
  for (int64_t p = 0; p < npair; ++p)
    for (int w = 0; w < 2; ++w) {
      int64_t r, c;
      order_tile(p, tm, tn, true, w, r, c);
      seen[(size_t)(r * tn + c)] = 1;
    }
  for (int64_t t = 0; t < 2 * npair; ++t) {
    int64_t r, c;
    order_tile(t, tm, tn, false, 0, r, c);
    if (!seen[(size_t)(r * tn + c)]) return false;
  }
  return true;
}

template <bool B_TERNARY, int OUT, bool RES = false>
hipError_t launch_two(const GemmArgs& g, int64_t row_bytes, int64_t tm, int64_t tn, int64_t npair,
                      int64_t rest, hipStream_t stream) {
  size_t lds = (size_t)kRing * Stage<B_TERNARY, true>::kBytes;
  lds = std::max(lds, (size_t)2 * kRing * Stage<B_TERNARY>::kBytes);
  lds = std::max(lds, kXchgBytes);
  auto kfn = gemm_mfma_two_kernel<B_TERNARY, OUT, RES>;
  hipError_t e =
      hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3((unsigned)(npair + rest)), dim3(2 * kWave), lds, stream, g.a_mask,
                     g.a_sign, g.a_alpha, g.b_mask, g.b_sign, g.b_alpha, g.M, g.N, row_bytes,
                     (int)tm, (int)tn, g.Y, g.ldy, (int)npair);
  return hipGetLastError();
}

template <bool B_TERNARY, int OUT, bool RES = false>
hipError_t launch_s(const GemmArgs& g, int S, int64_t row_bytes, int64_t tm, int64_t tn,
                    int64_t tile0, int64_t tiles, hipStream_t stream) {
  switch (S) {
    case 1:
      return launch_k<B_TERNARY, OUT, 1, RES>(g, row_bytes, tm, tn, tile0, tiles, stream);
    case 2:
      return launch_k<B_TERNARY, OUT, 2, RES>(g, row_bytes, tm, tn, tile0, tiles, stream);
    default:
      return launch_k<B_TERNARY, OUT, 4, RES>(g, row_bytes, tm, tn, tile0, tiles, stream);
  }
}

// Launches of one product, against the 1024 SIMDs (one wave each):
// * fewer than 1024 tiles: one launch, K split over S waves where that fills
//   more SIMDs (q, o, down of LLaMA-7B: 512 tiles, 30.5 us with S = 2 against
//   36.6 unsplit);
// * otherwise whole rounds of 1024 unsplit tiles, and a last partial round of
//   at most 512 tiles as a second launch with K split in two, which takes about
//   half as long as a round (LLaMA-7B q/k/v stacked: 1024 + 512 tiles);
// * batches and remainders above 512 unsplit: splitting every tile only adds
//   exchange work there (gate/up 80 us unsplit, 84 / 118 us with S = 2 / 4 on
//   every tile).
template <bool B_TERNARY, int OUT, bool RES = false>
hipError_t launch_plan(const GemmArgs& g, int64_t row_bytes, int64_t tm, int64_t tn,
                       hipStream_t stream) {
  const int64_t simds = 1024;
  const int64_t steps = (row_bytes / 8 + 3) / 4;
  const int64_t tiles = tm * tn;
  if (tiles * g.batch < simds)
    return launch_s<B_TERNARY, OUT, RES>(g, choose_split(tiles * g.batch, steps), row_bytes, tm,
                                         tn, 0, tiles, stream);
  const int64_t rem = tiles % simds;
  if (g.batch == 1 && rem > 0 && rem <= simds / 2 && steps >= 4) {
    // One launch for both parts where the pair order allows it (even column
    // count, whole column pairs in the first part, parts on 8-block boundaries).
    const int64_t npair = (tiles - rem) / 2;
    if (npair % 8 == 0 && pair_prefix_matches(tm, tn, npair))
      return launch_two<B_TERNARY, OUT, RES>(g, row_bytes, tm, tn, npair, rem, stream);
    const hipError_t e =
        launch_s<B_TERNARY, OUT, RES>(g, 1, row_bytes, tm, tn, 0, tiles - rem, stream);
    if (e != hipSuccess) return e;
    return launch_s<B_TERNARY, OUT, RES>(g, 2, row_bytes, tm, tn, tiles - rem, rem, stream);
  }
  // One unsplit launch: waves in pairs on adjacent column tiles, which load
  // their shared A panel once (a third fewer L2 requests and LDS bytes).
  if (tn >= 2)
    return launch_k<B_TERNARY, OUT, 1, RES, true>(g, row_bytes, tm, tn, 0, tm * ((tn + 1) / 2),
                                                  stream);
  return launch_s<B_TERNARY, OUT, RES>(g, 1, row_bytes, tm, tn, 0, tiles, stream);
}

template <bool B_TERNARY>
hipError_t launch_b(const GemmArgs& g, hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t tm = (g.M + WAVE_TILE - 1) / WAVE_TILE;
  const int64_t tn = (g.N + WAVE_TILE - 1) / WAVE_TILE;
  switch (g.y_dt) {
    case Elt::F32:
      return launch_plan<B_TERNARY, (int)Elt::F32>(g, row_bytes, tm, tn, stream);
    case Elt::BF16:
      return launch_plan<B_TERNARY, (int)Elt::BF16>(g, row_bytes, tm, tn, stream);
    default:
      return launch_plan<B_TERNARY, (int)Elt::I32>(g, row_bytes, tm, tn, stream);
  }
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream) {
  return g.b_mask ? launch_b<true>(g, stream) : launch_b<false>(g, stream);
}

// Two-plane product: g.N counts plane rows (twice the outputs), g.Y has g.N / 2
// columns; binary B, fp32 or bf16 output; K > 64 as for every launch of this
// kernel (the caller checks).
hipError_t launch_gemm_mfma_residual(const GemmArgs& g, hipStream_t stream) {
  if (g.b_mask || g.N % 64 != 0 || g.y_dt == Elt::I32) return hipErrorInvalidValue;
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t tm = (g.M + WAVE_TILE - 1) / WAVE_TILE;
  const int64_t tn = (g.N + WAVE_TILE - 1) / WAVE_TILE;
  // Launches as for one plane.
  return g.y_dt == Elt::F32 ? launch_plan<false, (int)Elt::F32, true>(g, row_bytes, tm, tn, stream)
                            : launch_plan<false, (int)Elt::BF16, true>(g, row_bytes, tm, tn, stream);
}

}  // namespace bwta
