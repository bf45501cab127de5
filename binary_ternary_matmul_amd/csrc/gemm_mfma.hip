// gemm_mfma.hip - binary x ternary and ternary x ternary products on the int8
// matrix cores of gfx950 (v_mfma_i32_16x16x64_i8, int32 accumulation).
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: a binary/ternary MatMul for the
// linear and the attention operators, on bit-packed operands.  The product is
//   acc[m][n] = sum_k t[m][k] * s[n][k],   t in {-1,0,+1}, s in {-1,+1} (or t),
// rescaled by alpha_a[m] * alpha_b[n] in the fused epilogue.
//
// Design (gfx950 first, not the page's CUDA kernel):
// * One wave owns a 128 x 128 output tile (8 x 8 MFMA tiles of 16 x 16, 256
//   int32 accumulators per lane, held in AGPRs at one wave per SIMD).
// * Operands stay packed until the last moment: each lane loads 64-bit words of
//   the mask/sign planes straight from global memory (L2-resident: a tile's
//   packed operands are 1/8 - 1/4 of their int8 size) and expands them in
//   registers directly into the MFMA operand layout.  No LDS is used for
//   operands.  The k order inside an MFMA is free as long as A and B use the
//   same one; lane group g = lane/16 takes the 64-bit word g of each 256-bit
//   step, and dword d (0..7) of a 32-bit word holds in byte j the bit 8j + d.
// * Expansion uses v_perm_b32 as a byte lookup (selector 0..7 picks a byte of
//   the 8-byte table, 12 gives 0x00, >= 13 gives 0xFF, 8 copies the sign of
//   byte 1):
//     binary  : sel = w & (0x01010101 << d)         table {+1, -1, -1, ., -1}
//     ternary : z  = (m & 0x0F0F0F0F) | ((s << 4) & 0xF0F0F0F0), and for the
//               upper nibbles z' = ((m >> 4) & 0x0F0F0F0F) | (s & 0xF0F0F0F0);
//               sel = z & (0x11111111 << i) for i = 0..2 and
//               (z >> 1) & 0x44444444 for i = 3       table {0, +1, +1, ., +1}
//   i.e. 2 VALU ops per 4 binary values and ~2.75 per 4 ternary values.
// * K is split over S waves of one block (S in {1, 2, 4}) when the grid would
//   otherwise leave SIMDs idle; the partial tiles are summed exactly in LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int TILES = 8;            // 16-row MFMA tiles per wave along M and along N
constexpr int WAVE_TILE = 16 * TILES;

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

template <bool B_TERNARY>
struct Packed {
  uint64_t am[TILES], as[TILES];
  uint64_t bm[B_TERNARY ? TILES : 1], bs[TILES];
};

// LDS staging of one step (256 k = 32 bytes of each of 128 rows per plane).
// Plane order in a stage: A mask, A sign, B sign, [B mask].
template <bool B_TERNARY>
struct Stage {
  static constexpr int kPlane = WAVE_TILE * 32;
  static constexpr int kPlanes = B_TERNARY ? 4 : 3;
  static constexpr int kBytes = kPlane * kPlanes;
};

// Copy 32 bytes of each of 128 rows of one plane into LDS with direct
// global->LDS 16-byte loads: lane i of instruction j moves half (i & 1) of row
// 32j + i/2, and the hardware stores lane i's 16 bytes at dst + 16 i, so row
// rho lands at dst + 32 rho.  Rows past `valid` reuse the last valid row (their
// results are never stored).  Only full steps (32 bytes inside the row) come
// here.
__device__ __forceinline__ void dma_plane(const uint8_t* __restrict__ plane, int64_t row_bytes,
                                          int valid, int64_t st, uint8_t* dst, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int rho = 32 * j + (lane >> 1);
    rho = rho < valid ? rho : valid - 1;
    const uint8_t* src = plane + (int64_t)rho * row_bytes + st * 32 + (lane & 1) * 16;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(dst + j * 1024), 16, 0, 0);
  }
}

template <bool B_TERNARY>
__device__ __forceinline__ void dma_step(const uint8_t* am, const uint8_t* as, const uint8_t* bm,
                                         const uint8_t* bs, int64_t row_bytes, int m_valid,
                                         int n_valid, int64_t st, uint8_t* stage, int lane) {
  constexpr int P = Stage<B_TERNARY>::kPlane;
  dma_plane(am, row_bytes, m_valid, st, stage, lane);
  dma_plane(as, row_bytes, m_valid, st, stage + P, lane);
  dma_plane(bs, row_bytes, n_valid, st, stage + 2 * P, lane);
  if constexpr (B_TERNARY) dma_plane(bm, row_bytes, n_valid, st, stage + 3 * P, lane);
}

// Lane (r, g) reads 64-bit word g of row 16t + r of each plane.
template <bool B_TERNARY>
__device__ __forceinline__ void read_stage(Packed<B_TERNARY>& p, const uint8_t* stage, int r,
                                           int g) {
  constexpr int P = Stage<B_TERNARY>::kPlane;
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int off = (16 * t + r) * 32 + 8 * g;
    p.am[t] = *reinterpret_cast<const uint64_t*>(stage + off);
    p.as[t] = *reinterpret_cast<const uint64_t*>(stage + P + off);
    p.bs[t] = *reinterpret_cast<const uint64_t*>(stage + 2 * P + off);
    if constexpr (B_TERNARY) p.bm[t] = *reinterpret_cast<const uint64_t*>(stage + 3 * P + off);
  }
}

// Partial last step (the row ends inside it): plain bounded loads.
template <bool B_TERNARY>
__device__ __forceinline__ void load_direct(Packed<B_TERNARY>& p, const uint8_t* __restrict__ am,
                                            const uint8_t* __restrict__ as,
                                            const uint8_t* __restrict__ bm,
                                            const uint8_t* __restrict__ bs, int64_t row_bytes,
                                            int64_t words, int64_t kw, int m_valid, int n_valid,
                                            int r) {
  const bool kin = kw < words;
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int ra = 16 * t + r < m_valid ? 16 * t + r : m_valid - 1;
    const int rb = 16 * t + r < n_valid ? 16 * t + r : n_valid - 1;
    const int64_t oa = (int64_t)ra * row_bytes + kw * 8;
    const int64_t ob = (int64_t)rb * row_bytes + kw * 8;
    p.am[t] = kin ? ld64(am + oa) : 0ull;
    p.as[t] = kin ? ld64(as + oa) : 0ull;
    p.bs[t] = kin ? ld64(bs + ob) : 0ull;
    if constexpr (B_TERNARY) p.bm[t] = kin ? ld64(bm + ob) : 0ull;
  }
}

template <bool B_TERNARY>
__device__ __forceinline__ void compute_step(const Packed<B_TERNARY>& p, v4i (&acc)[TILES][TILES]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      v4i a[TILES], b[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t)
        a[t] = expand_ternary((uint32_t)(p.am[t] >> (32 * h)), (uint32_t)(p.as[t] >> (32 * h)), q);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        if constexpr (B_TERNARY)
          b[t] = expand_ternary((uint32_t)(p.bm[t] >> (32 * h)), (uint32_t)(p.bs[t] >> (32 * h)), q);
        else
          b[t] = expand_binary((uint32_t)(p.bs[t] >> (32 * h)), q);
      }
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int j = 0; j < TILES; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
}

template <bool B_TERNARY, int OUT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_mfma_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                 const float* __restrict__ a_alpha, int64_t a_batch_rows,
                 const uint8_t* __restrict__ b_mask, const uint8_t* __restrict__ b_sign,
                 const float* __restrict__ b_alpha, int64_t b_batch_rows, int64_t M, int64_t N,
                 int64_t row_bytes, int tiles_n, void* __restrict__ Y, int64_t ldy,
                 int64_t y_batch_stride) {
  const int S = blockDim.x / kWave;
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;

  const int64_t b = blockIdx.z;
  const int tile_m = blockIdx.x / tiles_n;
  const int tile_n = blockIdx.x - tile_m * tiles_n;
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

  v4i acc[TILES][TILES];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int j = 0; j < TILES; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // Double-buffered LDS stages of this wave; step st+1 is in flight while step
  // st is expanded and multiplied.  Words past the row end (kw >= words) are
  // zeroed on the A side, which zeroes their products.
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stages = smem + (size_t)wid * 2 * Stage<B_TERNARY>::kBytes;
  // Full steps (32 bytes inside every row) go through the DMA pipeline; only
  // the very last step of a row can be partial, and it is peeled off so that
  // the loop body never waits on anything but its own stage.
  const int64_t full_steps = row_bytes / 32;
  const int64_t fe = st1 < full_steps ? st1 : (st0 > full_steps ? st0 : full_steps);
  if (st0 < fe) dma_step<B_TERNARY>(am, as, bm, bs, row_bytes, m_valid, n_valid, st0, stages, lane);
  for (int64_t st = st0; st < fe; ++st) {
    uint8_t* stage = stages + ((st - st0) & 1) * Stage<B_TERNARY>::kBytes;
    Packed<B_TERNARY> p;
    // vmcnt(0) (expcnt/lgkmcnt fields at their no-wait maxima): the DMA of this
    // step has landed in LDS.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    read_stage<B_TERNARY>(p, stage, r, g);
    if (st + 1 < fe)
      dma_step<B_TERNARY>(am, as, bm, bs, row_bytes, m_valid, n_valid, st + 1,
                          stages + ((st + 1 - st0) & 1) * Stage<B_TERNARY>::kBytes, lane);
    compute_step<B_TERNARY>(p, acc);
  }
  for (int64_t st = fe; st < st1; ++st) {  // at most one partial step
    Packed<B_TERNARY> p;
    const int64_t kw = st * 4 + g;
    load_direct<B_TERNARY>(p, am, as, bm, bs, row_bytes, words, kw, m_valid, n_valid, r);
    compute_step<B_TERNARY>(p, acc);
  }

  // Exact split-K reduction: waves 1..S-1 hand their tiles to wave 0 in turn
  // through one 64 KiB LDS slot (int32 addition is associative).
  v4i* red = reinterpret_cast<v4i*>(smem);
  if (S > 1) __syncthreads();  // every wave is done with its stages
  for (int src = 1; src < S; ++src) {
    if (wid == src) {
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int j = 0; j < TILES; ++j) red[(i * TILES + j) * kWave + lane] = acc[i][j];
    }
    __syncthreads();
    if (wid == 0) {
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int j = 0; j < TILES; ++j) acc[i][j] += red[(i * TILES + j) * kWave + lane];
    }
    __syncthreads();
  }
  if (wid != 0) return;

  // Epilogue: D[i][j] of a 16x16 tile sits in lane j + 16*(i/4), register i%4.
  float aa[TILES][4], ab[TILES];
  if constexpr (OUT != (int)Elt::I32) {
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 16 * i + 4 * g + q;
        aa[i][q] = row < m_valid ? a_alpha[a_row0 + row] : 0.0f;
      }
#pragma unroll
    for (int j = 0; j < TILES; ++j) {
      const int col = 16 * j + r;
      ab[j] = col < n_valid ? b_alpha[b_row0 + col] : 0.0f;
    }
  }
  char* ybase = static_cast<char*>(Y);
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 16 * i + 4 * g + q;
      if (row >= m_valid) continue;
      const int64_t yrow = b * y_batch_stride + (m0 + row) * ldy + n0;
#pragma unroll
      for (int j = 0; j < TILES; ++j) {
        const int col = 16 * j + r;
        if (col >= n_valid) continue;
        const int v = acc[i][j][q];
        if constexpr (OUT == (int)Elt::I32) {
          reinterpret_cast<int32_t*>(ybase)[yrow + col] = v;
        } else {
          const float sc = aa[i][q] * ab[j];
          const float y = (float)v * sc;
          if constexpr (OUT == (int)Elt::F32)
            reinterpret_cast<float*>(ybase)[yrow + col] = y;
          else
            reinterpret_cast<uint16_t*>(ybase)[yrow + col] = f32_to_bf16_rne(y);
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
  const size_t red_bytes = (size_t)TILES * TILES * kWave * sizeof(v4i);
  if (S > 1 && lds < red_bytes) lds = red_bytes;
#define BWTA_GEMM_LAUNCH(OUT_)                                                                  \
  do {                                                                                          \
    auto kfn = gemm_mfma_kernel<B_TERNARY, OUT_>;                                               \
    hipError_t e = hipFuncSetAttribute((const void*)kfn,                                        \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);   \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL(kfn, grid, block, lds, stream, g.a_mask, g.a_sign, g.a_alpha,            \
                       g.a_batch_rows, g.b_mask, g.b_sign, g.b_alpha, g.b_batch_rows, g.M, g.N, \
                       row_bytes, (int)tn, g.Y, g.ldy, g.y_batch_stride);                       \
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

hipError_t launch_gemm_mfma(const GemmArgs& g, hipStream_t stream) {
  return g.b_mask ? launch_b<true>(g, stream) : launch_b<false>(g, stream);
}

}  // namespace bwta
