// gemm_mfma_i8.hip - binary x ternary and ternary x ternary products on the
// int8 matrix cores of gfx950 (v_mfma_i32_32x32x32_i8, int32 accumulation):
// the int8 {-1, 0, +1} design, kept beside the FP4 kernel of gemm_mfma.hip
// (same sums, bit for bit) so that the two can be compared on the same data.
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: a binary/ternary MatMul for the
// linear and the attention operators, on bit-packed operands.  The product is
//   acc[m][n] = sum_k t[m][k] * s[n][k],   t in {-1,0,+1}, s in {-1,+1} (or t),
// rescaled by alpha_a[m] * alpha_b[n] in the fused epilogue.
//
// Design (gfx950 first, not the page's CUDA kernel):
// * One wave owns a 128 x 128 output tile (4 x 4 MFMA tiles of 32 x 32, 256
//   int32 accumulators per lane, held in AGPRs at one wave per SIMD; the
//   32 x 32 form keeps the register allocator from splitting them).
// * Operands stay packed until the last moment: the packed bit planes of each
//   256-k step (32 bytes per row) are copied global -> LDS with direct 16-byte
//   DMA loads, double-buffered per wave, and each lane expands the words it
//   needs from LDS in registers directly into the MFMA operand layout.  The k
//   order inside an MFMA is free as long as A and B use the same one: lane
//   group g = lane/32 takes 64-bit words 2g and 2g+1 of the step, and dword d
//   (0..7) of a 32-bit word holds in byte j the bit 8j + d.
// * Expansion uses v_perm_b32 as a byte lookup (selector 0..7 picks a byte of
//   the 8-byte table, 12 gives 0x00, >= 13 gives 0xFF).  Ternary x ternary
//   (attention scores) takes dword d (0..7) of a 32-bit word as byte j <- bit
//   8j + d of the nibble-interleaved mask/sign word z:
//     z  = (m & 0x0F0F0F0F) | ((s << 4) & 0xF0F0F0F0), and for the upper
//     nibbles z' = ((m >> 4) & 0x0F0F0F0F) | (s & 0xF0F0F0F0);
//     sel = z & (0x11111111 << i) for i = 0..2 and (z >> 1) & 0x44444444 for
//     i = 3, table {0, +1, +1, ., +1}.
//   Binary B uses a bit-slice k order in which the weight operand is a single
//   AND and the products carry a fixed scale (see expand_bitslice).
// * K is split over S waves of one block (S in {1, 2, 4}) when the grid would
//   otherwise leave SIMDs idle; the partial tiles are summed exactly in LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILES = 4;            // 32-row MFMA tiles per wave along M and along N
constexpr int WAVE_TILE = 32 * TILES;

// v_perm tables: __builtin_amdgcn_perm(hi, lo, sel) reads bytes 0..3 from lo
// and 4..7 from hi.
constexpr uint32_t kTernLo = 0x00010100u;  // byte0 = 0, bytes 1, 2 = +1
constexpr uint32_t kTernHi = 0x00000001u;  // byte4 = +1
constexpr uint32_t kBinLo = 0x00FFFF01u;   // byte0 = +1, bytes 1, 2 = -1
constexpr uint32_t kBinHi = 0x000000FFu;   // byte4 = -1

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Ternary operand for slice q (0: bits 8j+0..3, 1: bits 8j+4..7) of 32 k values.
__device__ __forceinline__ v4i expand_ternary(uint32_t m, uint32_t s, int q) {
  const uint32_t z = q == 0 ? ((m & 0x0F0F0F0Fu) | ((s << 4) & 0xF0F0F0F0u))
                            : (((m >> 4) & 0x0F0F0F0Fu) | (s & 0xF0F0F0F0u));
  v4i r;
  r[0] = (int)perm(kTernHi, kTernLo, z & 0x11111111u);
  r[1] = (int)perm(kTernHi, kTernLo, z & 0x22222222u);
  r[2] = (int)perm(kTernHi, kTernLo, z & 0x44444444u);
  r[3] = (int)perm(kTernHi, kTernLo, (z >> 1) & 0x44444444u);
  return r;
}

// Binary (+-1) operand for the same slice.
__device__ __forceinline__ v4i expand_binary(uint32_t w, int q) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (int)perm(kBinHi, kBinLo, w & (0x01010101u << (4 * q + i)));
  return r;
}

__device__ __forceinline__ uint64_t ld64(const uint8_t* p) {
  return *reinterpret_cast<const uint64_t*>(p);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Packed words of one step held by a lane: words 2g and 2g+1 of the rows
// 32t + r of each plane.
template <bool B_TERNARY>
struct Packed {
  uint64_t am[TILES][2], as[TILES][2];
  uint64_t bm[B_TERNARY ? TILES : 1][2], bs[TILES][2];
};

// LDS staging of one step (256 k = 32 bytes of each of 128 rows per plane).
// Plane order in a stage: A mask, A sign, B sign, [B mask].
template <bool B_TERNARY>
struct Stage {
  static constexpr int kPlane = WAVE_TILE * 32;
  static constexpr int kPlanes = B_TERNARY ? 4 : 3;
  static constexpr int kBytes = kPlane * kPlanes;
};

// Copy 32 bytes (one 256-k step) of each of 128 rows of one plane into LDS
// with direct global->LDS 16-byte loads: lane i of instruction j moves half
// (i & 1) of row 32j + i/2, and the hardware stores lane i's 16 bytes at
// dst + 16 i, so row rho lands at dst + 32 rho.  Every source stays inside the
// matrix:
// * rows past `valid` reuse the last valid row (their results are never stored);
// * a half that starts past the row end reads the row start instead (its words
//   are zeroed when the stage is read);
// * a half that straddles the row end (row_bytes % 16 == 8) reads the 16 bytes
//   that end at the row end, so the row's last word lands one word later in
//   the stage than its position; read_stage compensates.  This needs
//   row_bytes >= 16 (K > 64), which the launcher guarantees.
// The address is a wave-uniform base plus a 32-bit lane offset.
__device__ __forceinline__ void dma_plane(const uint8_t* __restrict__ plane, uint32_t row_bytes,
                                          int valid, uint32_t st, uint8_t* dst, int lane) {
  uint32_t o = st * 32 + (lane & 1) * 16;
  if (o + 16 > row_bytes) o = o < row_bytes ? row_bytes - 16 : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rho = min(32 * j + (lane >> 1), valid - 1);
    __builtin_amdgcn_global_load_lds(plane + ((uint32_t)rho * row_bytes + o),
                                     (lds_void_t*)(dst + j * 1024), 16, 0, 0);
  }
}

template <bool B_TERNARY>
__device__ __forceinline__ void dma_step(const uint8_t* am, const uint8_t* as, const uint8_t* bm,
                                         const uint8_t* bs, uint32_t row_bytes, int m_valid,
                                         int n_valid, uint32_t st, uint8_t* stage, int lane) {
  constexpr int P = Stage<B_TERNARY>::kPlane;
  dma_plane(am, row_bytes, m_valid, st, stage, lane);
  dma_plane(as, row_bytes, m_valid, st, stage + P, lane);
  dma_plane(bs, row_bytes, n_valid, st, stage + 2 * P, lane);
  if constexpr (B_TERNARY) dma_plane(bm, row_bytes, n_valid, st, stage + 3 * P, lane);
}

// Lane (r, g) reads 64-bit words 2g, 2g+1 of row 32t + r of each plane with one
// 16-byte LDS read.  `shift`: the row's last word straddled the DMA window and
// sits one slot late (it is word 2g, found in slot 2g+1).  Words past the row
// end are zeroed on the A side, which zeroes their products whatever B holds.
template <bool B_TERNARY>
__device__ __forceinline__ void read_stage(Packed<B_TERNARY>& p, const uint8_t* stage, int r,
                                           int g, bool shift, bool k0in, bool k1in) {
  constexpr int P = Stage<B_TERNARY>::kPlane;
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int off = (32 * t + r) * 32 + 16 * g;
    const u64x2 m = *reinterpret_cast<const u64x2*>(stage + off);
    const u64x2 s = *reinterpret_cast<const u64x2*>(stage + P + off);
    const u64x2 w = *reinterpret_cast<const u64x2*>(stage + 2 * P + off);
    p.am[t][0] = k0in ? (shift ? m[1] : m[0]) : 0ull;
    p.as[t][0] = k0in ? (shift ? s[1] : s[0]) : 0ull;
    p.am[t][1] = k1in ? m[1] : 0ull;
    p.as[t][1] = k1in ? s[1] : 0ull;
    p.bs[t][0] = shift ? w[1] : w[0];
    p.bs[t][1] = w[1];
    if constexpr (B_TERNARY) {
      const u64x2 bm = *reinterpret_cast<const u64x2*>(stage + 3 * P + off);
      p.bm[t][0] = shift ? bm[1] : bm[0];
      p.bm[t][1] = bm[1];
    }
  }
}

// One 256-k step: 8 slices of 32 k per lane group (word w, 32-bit half h,
// nibble half q).  The operands of slice s+1 are expanded while the 16 MFMAs of
// slice s run (two operand sets in flight), and the scheduler is asked to
// interleave that VALU work between the MFMAs.
template <bool B_TERNARY>
__device__ __forceinline__ void expand_slice(const Packed<B_TERNARY>& p, int sl, v4i (&a)[TILES],
                                             v4i (&b)[TILES]) {
  const int w = sl >> 2, h = (sl >> 1) & 1, q = sl & 1;
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    if constexpr (B_TERNARY)
      b[t] = expand_ternary((uint32_t)(p.bm[t][w] >> (32 * h)), (uint32_t)(p.bs[t][w] >> (32 * h)),
                            q);
    else
      b[t] = expand_binary((uint32_t)(p.bs[t][w] >> (32 * h)), q);
    a[t] = expand_ternary((uint32_t)(p.am[t][w] >> (32 * h)), (uint32_t)(p.as[t][w] >> (32 * h)),
                          q);
  }
}

template <bool B_TERNARY>
__device__ __forceinline__ void compute_step_tt(const Packed<B_TERNARY>& p,
                                                v16i (&acc)[TILES][TILES]) {
  v4i a[2][TILES], b[2][TILES];
  expand_slice<B_TERNARY>(p, 0, a[0], b[0]);
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) {
    const int cur = sl & 1;
    if (sl + 1 < 8) expand_slice<B_TERNARY>(p, sl + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int j = 0; j < TILES; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
    // 16 MFMAs, each followed by a share of the next slice's expansion VALU.
#pragma unroll
    for (int k = 0; k < TILES * TILES; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // up to 6 VALU
    }
  }
}

// Binary B in bit-slice order.  Slice d (0..7) takes, in dword x (0..3) byte j,
// the bit 8j + d of the lane's 32-bit word x, for A and for B alike (the k order
// inside an MFMA is free as long as both sides agree).  The weight operand is
// then a single AND: bytes {0, 2^d} = b * 2^d with b = 1 for a negative weight
// (bit 7 is moved to bit 6 and counted with 2^6).  The activation operand
// t * 2^(6-d) (2^0 for d = 7) comes from a v_perm lookup whose table absorbs the
// scale, so every product is 64 t b and
//   acc64 = 64 sum t b,   sum t s = sum t (1 - 2b) = rowsum(t) - acc64 / 32,
// with rowsum(t) = nnz - 2 popc(sign).  Per slice and tile: 4 ANDs for B, 4
// shift+mask selectors and 4 lookups for A, against 16 lookups + 12 ops before.
__device__ __forceinline__ uint32_t bs_table(int d) {
  const uint32_t c = 1u << (6 - (d < 6 ? d : 6));
  return ((0u - c) & 0xFFu) << 24 | c << 8;  // byte0 = 0, byte1 = +c, byte3 = -c
}

// A words with (mask, sign) bit pairs adjacent: u holds the even bits, v the odd.
struct BitSliceA {
  uint32_t u[TILES][4], v[TILES][4];
};

__device__ __forceinline__ void prep_bitslice(const Packed<false>& p, BitSliceA& q) {
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t m = (uint32_t)(p.am[t][x >> 1] >> (32 * (x & 1)));
      const uint32_t s = (uint32_t)(p.as[t][x >> 1] >> (32 * (x & 1)));
      q.u[t][x] = (m & 0x55555555u) | ((s << 1) & 0xAAAAAAAAu);
      q.v[t][x] = ((m >> 1) & 0x55555555u) | (s & 0xAAAAAAAAu);
    }
}

__device__ __forceinline__ void expand_bitslice(const Packed<false>& p, const BitSliceA& q, int d,
                                                v4i (&a)[TILES], v4i (&b)[TILES]) {
  const uint32_t tab = bs_table(d);
  const int sh = d & ~1;
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t src = (d & 1) ? q.v[t][x] : q.u[t][x];
      a[t][x] = (int)perm(0u, tab, (src >> sh) & 0x03030303u);
      const uint32_t w = (uint32_t)(p.bs[t][x >> 1] >> (32 * (x & 1)));
      b[t][x] = (int)(d < 7 ? (w & (0x01010101u << d)) : ((w >> 1) & 0x40404040u));
    }
}

__device__ __forceinline__ void compute_step_bin(const Packed<false>& p, v16i (&acc)[TILES][TILES],
                                                 int (&pop)[TILES]) {
  BitSliceA q;
  prep_bitslice(p, q);
#pragma unroll
  for (int t = 0; t < TILES; ++t)
    pop[t] += __builtin_popcountll(p.as[t][0]) + __builtin_popcountll(p.as[t][1]);
  v4i a[2][TILES], b[2][TILES];
  expand_bitslice(p, q, 0, a[0], b[0]);
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int cur = d & 1;
    if (d + 1 < 8) expand_bitslice(p, q, d + 1, a[cur ^ 1], b[cur ^ 1]);
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int j = 0; j < TILES; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < TILES * TILES; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to 4 VALU
    }
  }
}

// Output tile in LDS: 128 rows of 128 int32, padded by 8 words per row so that
// the accumulator writes (2 rows x 32 columns per instruction, 4 rows apart)
// hit 64 distinct banks.
constexpr int kTileLd = WAVE_TILE + 8;
constexpr size_t kTileBytes = (size_t)WAVE_TILE * kTileLd * 4;

template <bool B_TERNARY, int OUT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_mfma_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                 const float* __restrict__ a_alpha, const int32_t* __restrict__ a_nnz,
                 int64_t a_batch_rows,
                 const uint8_t* __restrict__ b_mask, const uint8_t* __restrict__ b_sign,
                 const float* __restrict__ b_alpha, int64_t b_batch_rows, int64_t M, int64_t N,
                 int64_t row_bytes, int tiles_m, int tiles_n, void* __restrict__ Y, int64_t ldy,
                 int64_t y_batch_stride) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int S = blockDim.x / kWave;
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int r = lane & 31;
  const int g = lane >> 5;

  // Blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
  // of tiles (consecutive tile_n for the same tile_m) so that tiles sharing A
  // rows share that XCD's L2.
  const int nblk = tiles_m * tiles_n;
  int lin = blockIdx.x;
  if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int tile_m = lin / tiles_n;
  const int tile_n = lin - tile_m * tiles_n;
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
  const int64_t st0 = steps * wid / S;
  const int64_t st1 = steps * (wid + 1) / S;

  // The tile's scales go to LDS now; the loads complete behind the main loop
  // and the epilogue reads them from LDS (made visible by its first barrier).
  __shared__ float s_alpha_a[WAVE_TILE], s_alpha_b[WAVE_TILE];
  __shared__ int s_rowsum[B_TERNARY ? 1 : WAVE_TILE];  // nnz, then nnz - 2 popc(sign)
  if constexpr (!B_TERNARY) {
    if (wid == 0) {
#pragma unroll
      for (int h = 0; h < WAVE_TILE / kWave; ++h) {
        const int i = h * kWave + lane;
        s_rowsum[i] = i < m_valid ? a_nnz[b * a_batch_rows + m0 + i] : 0;
      }
    }
  }
  if constexpr (OUT != (int)Elt::I32) {
    if (wid == 0) {
#pragma unroll
      for (int h = 0; h < WAVE_TILE / kWave; ++h) {
        const int i = h * kWave + lane;
        s_alpha_a[i] = i < m_valid ? a_alpha[b * a_batch_rows + m0 + i] : 0.0f;
        s_alpha_b[i] = i < n_valid ? b_alpha[b * b_batch_rows + n0 + i] : 0.0f;
      }
    }
  }

  v16i acc[TILES][TILES];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int j = 0; j < TILES; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

  // Double-buffered LDS stages of this wave: step st+1 is in flight while step
  // st is expanded and multiplied.
  int pop[TILES] = {0, 0, 0, 0};  // popc(sign) of this lane's words of rows 32t + r
  uint8_t* stages = smem + (size_t)wid * 2 * Stage<B_TERNARY>::kBytes;
  const uint32_t rb = (uint32_t)row_bytes;
  const bool straddle = (rb & 15u) == 8u;  // the last word is read one slot late
  if (st0 < st1) dma_step<B_TERNARY>(am, as, bm, bs, rb, m_valid, n_valid, (uint32_t)st0, stages, lane);
  for (int64_t st = st0; st < st1; ++st) {
    uint8_t* stage = stages + ((st - st0) & 1) * Stage<B_TERNARY>::kBytes;
    Packed<B_TERNARY> p;
    // vmcnt(0) (expcnt/lgkmcnt fields at their no-wait maxima): the DMA of this
    // step has landed in LDS.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (st * 4 + 4 <= words) {
      read_stage<B_TERNARY>(p, stage, r, g, false, true, true);
    } else {  // the row ends inside this step
      const int64_t kw = st * 4 + 2 * g;
      read_stage<B_TERNARY>(p, stage, r, g, straddle && kw == words - 1, kw < words,
                            kw + 1 < words);
    }
    if (st + 1 < st1)
      dma_step<B_TERNARY>(am, as, bm, bs, rb, m_valid, n_valid, (uint32_t)(st + 1),
                          stages + ((st + 1 - st0) & 1) * Stage<B_TERNARY>::kBytes, lane);
    if constexpr (B_TERNARY)
      compute_step_tt<B_TERNARY>(p, acc);
    else
      compute_step_bin(p, acc, pop);
  }

  // Sum the S partial tiles exactly in one LDS tile (wave 0 stores, the others
  // add with LDS integer atomics), then let all S waves write the result.
  // D[i][j] of a 32x32 MFMA tile sits in lane j + 32*((i/4)%2), register
  // (i%4) + 4*(i/8).
  int32_t* tile = reinterpret_cast<int32_t*>(smem);
  __syncthreads();  // every wave is done with its stages; staged scales are visible
  if constexpr (!B_TERNARY) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int both = pop[t] + __shfl_xor(pop[t], 32, kWave);  // the two lane groups
      if (g == 0) atomicAdd(&s_rowsum[32 * t + r], -2 * both);
    }
  }
  if (wid == 0) {
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int j = 0; j < TILES; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q)
          tile[(32 * i + (q & 3) + 8 * (q >> 2) + 4 * g) * kTileLd + 32 * j + r] = acc[i][j][q];
  }
  if (S > 1) {
    __syncthreads();
    if (wid != 0) {
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int j = 0; j < TILES; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q)
            atomicAdd(&tile[(32 * i + (q & 3) + 8 * (q >> 2) + 4 * g) * kTileLd + 32 * j + r],
                      acc[i][j][q]);
    }
  }
  __syncthreads();

  // Epilogue: each wave takes rows wid, wid + S, ...; a half-wave covers one
  // 128-column row with 4 columns per lane, so every store is row-contiguous
  // (one 16- or 8-byte store per lane when the row is aligned and complete).
  const int half = lane >> 5;
  const int c4 = (lane & 31) * 4;
  float ab[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (OUT != (int)Elt::I32) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ab[u] = s_alpha_b[c4 + u];
  }
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  const bool vec_ok = ((ldy * ES) % 16 == 0) && ((y_batch_stride * ES) % 16 == 0) &&
                      ((n0 * ES) % 16 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0);
  const bool full_cols = c4 + 4 <= n_valid;
  char* ybase = static_cast<char*>(Y);
  for (int row = 2 * wid + half; row < m_valid; row += 2 * S) {
    int4 v = *reinterpret_cast<const int4*>(&tile[row * kTileLd + c4]);
    if constexpr (!B_TERNARY) {
      // bit-slice accumulators hold 64 sum t b: sum t s = rowsum - acc / 32
      const int rs = s_rowsum[row];
      v.x = rs - (v.x >> 5);
      v.y = rs - (v.y >> 5);
      v.z = rs - (v.z >> 5);
      v.w = rs - (v.w >> 5);
    }
    const int vv[4] = {v.x, v.y, v.z, v.w};
    const int64_t yoff = b * y_batch_stride + (m0 + row) * ldy + n0 + c4;
    if constexpr (OUT == (int)Elt::I32) {
      int32_t* y = reinterpret_cast<int32_t*>(ybase) + yoff;
      if (vec_ok && full_cols) {
        *reinterpret_cast<int4*>(y) = v;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c4 + u < n_valid) y[u] = vv[u];
      }
    } else {
      const float aa = s_alpha_a[row];
      float out[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float sc = aa * ab[u];
        out[u] = (float)vv[u] * sc;
      }
      if constexpr (OUT == (int)Elt::F32) {
        float* y = reinterpret_cast<float*>(ybase) + yoff;
        if (vec_ok && full_cols) {
          *reinterpret_cast<float4*>(y) = make_float4(out[0], out[1], out[2], out[3]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c4 + u < n_valid) y[u] = out[u];
        }
      } else {
        uint16_t* y = reinterpret_cast<uint16_t*>(ybase) + yoff;
        uint16_t h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) h[u] = f32_to_bf16_rne(out[u]);
        if (vec_ok && full_cols) {
          *reinterpret_cast<uint2*>(y) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                                    (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c4 + u < n_valid) y[u] = h[u];
        }
      }
    }
  }
}

// Split K over S waves when that fills more SIMDs: minimise rounds(S) / S, where a
// round is one wave on each of the 1024 SIMDs; keep >= 2 steps per wave.
int choose_split(int64_t tiles, int64_t steps) {
  const int64_t simds = 1024;
  int best = 1;
  double best_cost = 1e30;
  for (int S = 1; S <= 4; S *= 2) {
    if (S > 1 && steps / S < 2) break;
    const double rounds = (double)((tiles * S + simds - 1) / simds);
    const double cost = rounds / S;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

template <bool B_TERNARY>
hipError_t launch_b(const GemmArgs& g, hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t tm = (g.M + WAVE_TILE - 1) / WAVE_TILE;
  const int64_t tn = (g.N + WAVE_TILE - 1) / WAVE_TILE;
  const int64_t steps = (row_bytes / 8 + 3) / 4;
  const int S = choose_split(tm * tn * g.batch, steps);
  const dim3 grid((unsigned)(tm * tn), 1, (unsigned)g.batch);
  const dim3 block((unsigned)(S * kWave));
  size_t lds = (size_t)S * 2 * Stage<B_TERNARY>::kBytes;
  if (lds < kTileBytes) lds = kTileBytes;
#define BWTA_GEMM_LAUNCH(OUT_)                                                                  \
  do {                                                                                          \
    auto kfn = gemm_mfma_kernel<B_TERNARY, OUT_>;                                               \
    hipError_t e = hipFuncSetAttribute((const void*)kfn,                                        \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);   \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL(kfn, grid, block, lds, stream, g.a_mask, g.a_sign, g.a_alpha,            \
                       g.a_nnz, g.a_batch_rows, g.b_mask, g.b_sign, g.b_alpha, g.b_batch_rows, g.M, g.N, \
                       row_bytes, (int)tm, (int)tn, g.Y, g.ldy, g.y_batch_stride);                       \
  } while (0)
  switch (g.y_dt) {
    case Elt::F32:
      BWTA_GEMM_LAUNCH((int)Elt::F32);
      break;
    case Elt::BF16:
      BWTA_GEMM_LAUNCH((int)Elt::BF16);
      break;
    case Elt::I32:
      BWTA_GEMM_LAUNCH((int)Elt::I32);
      break;
  }
#undef BWTA_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma_i8(const GemmArgs& g, hipStream_t stream) {
  return g.b_mask ? launch_b<true>(g, stream) : launch_b<false>(g, stream);
}

}  // namespace bwta
