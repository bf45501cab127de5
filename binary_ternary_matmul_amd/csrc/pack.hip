// pack.hip - online ternarization and weight binarization with bit packing.
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: activations become ternary by
// projecting tiny values to zero, weights become binary, and both are
// bit-packed (Figure 6 shows 32 values packed into one 32-bit word).  The
// threshold and the scales follow the library definition in bwta.h:
//   mu = tree(|x|)/K, thr = 0.5*mu, t = |x| <= thr ? 0 : sign(x),
//   alpha_a = tree(kept |x|)/nnz;  alpha_w = tree(|w|)/K, s = (w < 0) ? -1 : +1.
//
// Layout of the work.  A row is cut into groups of G = 64*V elements, V = 16
// bytes / element size (4 fp32 or 8 bf16).  In group i lane l owns the V
// consecutive elements [i*G + l*V, +V), which it reads with one 16-byte load,
// so every wave-wide load is one contiguous 1 KiB run.  A wave owns GPW
// consecutive groups (GPW a power of two); W waves share a row when
// GPW*G*W >= K needs them, and every (lane run, group, wave) block is an aligned
// power-of-two sub-tree of the tree over the zero-padded row, so
//   lane tree (V) -> wave tree (64 lanes x GPW groups) -> LDS tree (W waves)
// reproduces the definition bit for bit.  The row stays in registers between
// the two passes (sum, then threshold), so x is read from HBM once.
//
// Bits: lane l's V mask/sign bits land at bit offset l*V of its group; lanes are
// OR-combined with shuffles into 32-bit words (8 lanes of 4 bits for fp32, 4
// lanes of 8 bits for bf16) and stored as whole words.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int V = 4;
  static constexpr int GPW_MAX = 16;
};
template <>
struct Elem<uint16_t> {
  static constexpr int V = 8;
  static constexpr int GPW_MAX = 8;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_bits_to_f32(v); }

// V elements starting at k = e of one row (zeros beyond K).
template <typename T, bool VEC>
__device__ __forceinline__ void load_run(const T* __restrict__ row, int64_t e, int64_t K,
                                         int64_t sk, float (&out)[Elem<T>::V]) {
  constexpr int V = Elem<T>::V;
  if (VEC && e + V <= K) {
    const u32x4 u = load_nt16(row + e);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = __uint_as_float(w[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[2 * j] = bf16_bits_to_f32(w[j] & 0xFFFFu);
        out[2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) out[j] = (e + j < K) ? to_f32(row[(e + j) * sk]) : 0.0f;
  }
}

// One row (or W rows' worth of waves) per iteration; see the file comment.
template <typename T, int GPW, bool TERNARY, bool VEC>
__global__ void __launch_bounds__(1024)
pack_rows_kernel(const T* __restrict__ X, int64_t rows, int64_t K, int64_t sr, int64_t sk, int W,
                 int64_t row_bytes, uint8_t* __restrict__ mask, uint8_t* __restrict__ sign,
                 float* __restrict__ alpha, int32_t* __restrict__ nnz) {
  constexpr int V = Elem<T>::V;
  constexpr int G = kWave * V;
  constexpr int LPW = 32 / V;  // lanes per 32-bit output word
  __shared__ float red_sum[16];
  __shared__ float red_kept[16];
  __shared__ int red_cnt[16];

  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int rpb = (blockDim.x / kWave) / W;
  const int row_in_block = wid / W;
  const int w_in_row = wid - row_in_block * W;
  const int64_t Kp = row_bytes * 8;
  const float fK = (float)K;

  for (int64_t r0 = (int64_t)blockIdx.x * rpb; r0 < rows; r0 += (int64_t)gridDim.x * rpb) {
    const int64_t r = r0 + row_in_block;
    const bool live = r < rows;
    const T* xrow = X + (live ? r : 0) * sr;

    float x[GPW][V];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int64_t e = (int64_t)(w_in_row * GPW + i) * G + (int64_t)lane * V;
      if (live) {
        load_run<T, VEC>(xrow, e, K, sk, x[i]);
      } else {
#pragma unroll
        for (int j = 0; j < V; ++j) x[i][j] = 0.0f;
      }
    }

    // Pass 1: tree(|x|).
    float part[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      float a[V];
#pragma unroll
      for (int j = 0; j < V; ++j) a[j] = fabsf(x[i][j]);
      part[i] = lane_tree<V>(a);
    }
    float total = wave_tree<GPW>(part);
    if (W > 1) {
      if (lane == 0) red_sum[wid] = total;
      __syncthreads();
      total = tree16(&red_sum[row_in_block * W], W);
    }

    uint32_t mbits[GPW], sbits[GPW];
    float alpha_v;
    int count = 0;
    if constexpr (TERNARY) {
      const float mu = total / fK;
      const float thr = 0.5f * mu;
      // Pass 2: threshold, planes, tree(kept |x|), nnz.
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        float kept[V];
        uint32_t mb = 0, sb = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float a = fabsf(x[i][j]);
          const bool keep = a > thr;
          kept[j] = keep ? a : 0.0f;
          mb |= (uint32_t)keep << j;
          sb |= (uint32_t)(keep && x[i][j] < 0.0f) << j;
        }
        part[i] = lane_tree<V>(kept);
        mbits[i] = mb;
        sbits[i] = sb;
        count += __builtin_popcount(mb);
      }
      float ktot = wave_tree<GPW>(part);
      int ctot = wave_sum_int(count);
      if (W > 1) {
        if (lane == 0) {
          red_kept[wid] = ktot;
          red_cnt[wid] = ctot;
        }
        __syncthreads();
        ktot = tree16(&red_kept[row_in_block * W], W);
        ctot = 0;
        for (int q = 0; q < W; ++q) ctot += red_cnt[row_in_block * W + q];
      }
      count = ctot;
      alpha_v = ctot ? ktot / (float)ctot : 0.0f;
    } else {
      alpha_v = total / fK;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        uint32_t sb = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) sb |= (uint32_t)(x[i][j] < 0.0f) << j;
        sbits[i] = sb;
        mbits[i] = 0;
      }
    }

    // Combine LPW lanes into one 32-bit word per plane and store it.
    const int64_t base = (live ? r : 0) * row_bytes;
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      uint32_t m = mbits[i], s = sbits[i];
#pragma unroll
      for (int d = 1; d < LPW; d <<= 1) {
        if constexpr (TERNARY) m |= (uint32_t)__shfl_down((int)m, d, kWave) << (d * V);
        s |= (uint32_t)__shfl_down((int)s, d, kWave) << (d * V);
      }
      const int64_t bit = (int64_t)(w_in_row * GPW + i) * G + (int64_t)lane * V;
      if (live && (lane % LPW) == 0 && bit < Kp) {
        if constexpr (TERNARY) *reinterpret_cast<uint32_t*>(mask + base + bit / 8) = m;
        *reinterpret_cast<uint32_t*>(sign + base + bit / 8) = s;
      }
    }
    if (live && w_in_row == 0 && lane == 0) {
      alpha[r] = alpha_v;
      if constexpr (TERNARY) nnz[r] = count;
    }
  }
}

struct Plan {
  int gpw;    // groups per wave
  int W;      // waves per row
  int wpb;    // waves per block
};

template <typename T>
Plan plan_for(int64_t K) {
  constexpr int G = kWave * Elem<T>::V;
  int64_t n = (K + G - 1) / G;
  int64_t p = 1;
  while (p < n) p <<= 1;
  Plan pl;
  pl.gpw = (int)(p < Elem<T>::GPW_MAX ? p : Elem<T>::GPW_MAX);
  pl.W = (int)(p / pl.gpw);
  pl.wpb = pl.W >= 4 ? pl.W : 4;
  return pl;
}

template <typename T, bool TERNARY, bool VEC>
hipError_t launch_typed(const T* X, int64_t rows, int64_t K, int64_t sr, int64_t sk, uint8_t* mask,
                        uint8_t* sign, float* alpha, int32_t* nnz, hipStream_t stream) {
  const Plan pl = plan_for<T>(K);
  const int64_t row_bytes = (K + 63) / 64 * 8;
  const int rpb = pl.wpb / pl.W;
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  const dim3 grid((unsigned)blocks), block((unsigned)(pl.wpb * kWave));
#define BWTA_PACK_CASE(G_)                                                                     \
  case G_:                                                                                     \
    if constexpr (G_ <= Elem<T>::GPW_MAX)                                                      \
      hipLaunchKernelGGL((pack_rows_kernel<T, G_, TERNARY, VEC>), grid, block, 0, stream, X,   \
                         rows, K, sr, sk, pl.W, row_bytes, mask, sign, alpha, nnz);            \
    break;
  switch (pl.gpw) {
    BWTA_PACK_CASE(1)
    BWTA_PACK_CASE(2)
    BWTA_PACK_CASE(4)
    BWTA_PACK_CASE(8)
    BWTA_PACK_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef BWTA_PACK_CASE
  return hipGetLastError();
}

template <bool TERNARY>
hipError_t launch_any(const void* X, Elt dt, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                      uint8_t* mask, uint8_t* sign, float* alpha, int32_t* nnz, hipStream_t stream) {
  const size_t es = dt == Elt::F32 ? 4 : 2;
  const bool vec = sk == 1 && (reinterpret_cast<uintptr_t>(X) % 16 == 0) &&
                   ((sr * (int64_t)es) % 16 == 0 || rows <= 1);
  if (dt == Elt::F32) {
    auto p = static_cast<const float*>(X);
    return vec ? launch_typed<float, TERNARY, true>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream)
               : launch_typed<float, TERNARY, false>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream);
  }
  auto p = static_cast<const uint16_t*>(X);
  return vec ? launch_typed<uint16_t, TERNARY, true>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream)
             : launch_typed<uint16_t, TERNARY, false>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream);
}

}  // namespace

hipError_t launch_ternarize(const void* X, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                            uint8_t* mask, uint8_t* sign, float* alpha, int32_t* nnz,
                            hipStream_t stream) {
  return launch_any<true>(X, dt, rows, K, stride_row, 1, mask, sign, alpha, nnz, stream);
}

hipError_t launch_binarize(const void* W, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                           int64_t stride_k, uint8_t* sign, float* alpha, hipStream_t stream) {
  return launch_any<false>(W, dt, rows, K, stride_row, stride_k, nullptr, sign, alpha, nullptr,
                           stream);
}

}  // namespace bwta
