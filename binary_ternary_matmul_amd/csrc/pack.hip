// pack.hip - online ternarization and weight binarization with bit packing.
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: activations become ternary by
// projecting tiny values to zero, weights become binary, and both are
// bit-packed (Figure 6 packs 32 values into one 32-bit word).  The threshold and
// the scales follow the library definition in bwta.h:
//   mu = tree(|x|)/K, thr = 0.5*mu, t = |x| <= thr ? 0 : sign(x),
//   alpha_a = tree(kept |x|)/nnz;  alpha_w = tree(|w|)/K, s = (w < 0) ? -1 : +1.
//
// Row kernel.  A row is cut into groups of G = LPR*8 elements; in a group, lane
// l (of the LPR lanes serving the row) owns the 8 consecutive elements
// [8l, 8l+8), read with one (bf16) or two (fp32) 16-byte loads, so a wave-wide
// load is one contiguous run.  Those 8 elements give exactly one byte of each
// bit plane, which the lane stores itself: no cross-lane bit shuffling.  A wave
// owns GPW consecutive groups; W waves share a row when one wave is not enough.
// Every (lane run, group, wave) block is an aligned power-of-two sub-tree of the
// tree over the zero-padded row, so
//   lane tree (8) -> wave tree (LPR lanes x GPW groups) -> LDS tree (W waves)
// reproduces the definition bit for bit.  Small rows (K <= 256) use LPR = 16 or
// 32 lanes per row, several rows per wave.  The row stays in registers between
// the two passes (sum, then threshold), so x is read from HBM once.
//
// Column kernels.  Packing the columns of a row-major [K, C] matrix (V^T for
// attention) gives each lane one column, folds its column's aligned runs into
// the pairwise tree with a register stack (a binary counter over the run
// index), and lets 16 waves split K into aligned power-of-two ranges.  The
// staged kernel brings 64 KiB tiles through LDS with 16-byte loads (one
// memory round trip per 16 x 32 rows, the next tile in flight); the per-lane
// kernel, for the remaining shapes, reads its column element by element.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

constexpr int RUN = 8;  // elements per lane run = bits per stored plane byte

// Workgroup barrier ordering LDS only (global loads in flight are not awaited).
__device__ __forceinline__ void lds_barrier_local() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
struct Raw {
  static constexpr int kWords = RUN * (int)sizeof(T) / 4;  // 32-bit words per run
};

// fp32 bit pattern of element j of a run.
__device__ __forceinline__ uint32_t ebits(const uint32_t* raw, int j, float) { return raw[j]; }
__device__ __forceinline__ uint32_t ebits(const uint32_t* raw, int j, uint16_t) {
  return (raw[j >> 1] >> (16 * (j & 1))) << 16;
}

// Decisions as integer arithmetic on the IEEE bit patterns (finite inputs), so
// no per-element lane masks are formed.  For non-negative floats a, t:
// a > t  <=>  bits(a) > bits(t)  <=>  bit 31 of (bits(t) - bits(a)).
__device__ __forceinline__ uint32_t gt_bit(uint32_t ua, uint32_t ut) { return (ut - ua) >> 31; }
// x < 0 (so -0.0 counts as non-negative): sign bit set and not exactly -0.0.
__device__ __forceinline__ uint32_t neg_bit(uint32_t ux) {
  return (ux >> 31) & ((0x80000000u - ux) >> 31);
}

// bf16 pass 2 on packed 16-bit halves.  A run word holds elements 2q (low
// half) and 2q+1 (high half).  A bf16 value widens to fp32 exactly (low 16 bits
// zero), so for a finite non-negative threshold with fp32 bit pattern U,
// |x| > thr  <=>  bits16(|x|) > U >> 16: one 16-bit subtraction per half decides
// two elements, and its sign bit spread over the half is the keep mask.  Bit
// 2q of the low half and bit 2q+1 of the high half collect the mask and the
// sign bits; folding the halves gives the plane bytes.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void ternary_run_bf16(const uint32_t (&raw)[4], uint32_t t2, float& ksum,
                                                 uint32_t& mb, uint32_t& sb, uint32_t& cnt) {
  float kept[RUN];
  uint32_t macc = 0, nacc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t a = raw[q] & 0x7FFF7FFFu;  // |x| of both halves
    const u16x2 d = __builtin_bit_cast(u16x2, t2) - __builtin_bit_cast(u16x2, a);
    const uint32_t km = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, d) >> (int16_t)15);
    const uint32_t kw = a & km;  // kept |x| (or +0) of both halves
    kept[2 * q] = __uint_as_float(kw << 16);
    kept[2 * q + 1] = __uint_as_float(kw & 0xFFFF0000u);
    const uint32_t place = (1u << (2 * q)) | (2u << (16 + 2 * q));
    macc |= km & place;
    const u16x2 neg = __builtin_bit_cast(u16x2, raw[q]) >>
                      u16x2{(uint16_t)(15 - 2 * q), (uint16_t)(14 - 2 * q)};
    nacc |= __builtin_bit_cast(uint32_t, neg) & place;
  }
  ksum = lane_tree<RUN>(kept);
  cnt = __builtin_popcount(macc);
  mb = macc | (macc >> 16);
  sb = mb & (nacc | (nacc >> 16));
}

__device__ __forceinline__ uint32_t raw_bits(float v) { return __float_as_uint(v); }
__device__ __forceinline__ uint32_t raw_bits(uint16_t v) { return v; }

// The run of 8 elements starting at k = e of one row, as raw words.
// MODE 0: the run lies inside the row, unit stride, 16-byte aligned: vector
//         loads, issued back to back by the caller for all its runs.
// MODE 1: unit stride, aligned, K a multiple of 8, so a run lies either inside
//         the row (vector load) or past its end (zeros).
// MODE 2: any strides (the generic gather): element loads, 64-bit offsets.
template <typename T, int MODE>
__device__ __forceinline__ void load_run(const T* __restrict__ row, int64_t e, int64_t K,
                                         int64_t sk, uint32_t (&raw)[Raw<T>::kWords]) {
  constexpr int NW = Raw<T>::kWords;
  auto vec = [&](int32_t off) {
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) {
      const u32x4 u = load_nt16(row + off + v * (16 / sizeof(T)));
      raw[4 * v + 0] = u.x;
      raw[4 * v + 1] = u.y;
      raw[4 * v + 2] = u.z;
      raw[4 * v + 3] = u.w;
    }
  };
  auto put = [&](int j, uint32_t b) {
    if constexpr (sizeof(T) == 4)
      raw[j] = b;
    else
      raw[j >> 1] |= b << (16 * (j & 1));
  };
  if constexpr (MODE == 0) {
    vec((int32_t)e);
  } else if constexpr (MODE == 1) {
    if (e < K) {
      vec((int32_t)e);
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) raw[w] = 0u;
    }
  } else {
#pragma unroll
    for (int w = 0; w < NW; ++w) raw[w] = 0u;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int64_t k = e + j < K ? e + j : K - 1;
      const uint32_t b = raw_bits(row[k * sk]);
      put(j, e + j < K ? b : 0u);
    }
  }
}

// The run of 8 elements at byte offset voff + soff of a row descriptor, with
// 16-byte non-temporal buffer loads: a run past the descriptor's range reads
// zeros (rows whose length is a multiple of 8 and 16-byte aligned, so a run is
// wholly inside or wholly outside).
constexpr int kNonTemporal = 2;  // buffer cache-policy bits: nt
template <typename T>
__device__ __forceinline__ void load_run_buf(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                             uint32_t (&raw)[Raw<T>::kWords]) {
  constexpr int NW = Raw<T>::kWords;
#pragma unroll
  for (int v = 0; v < NW / 4; ++v) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * v, soff, kNonTemporal);
    raw[4 * v + 0] = u.x;
    raw[4 * v + 1] = u.y;
    raw[4 * v + 2] = u.z;
    raw[4 * v + 3] = u.w;
  }
}

template <int LPR>
__device__ __forceinline__ float lanes_tree(float v) {
  // pairwise over the LPR lanes of one row (lane bit 0 first)
#pragma unroll
  for (int b = 1; b < LPR; b <<= 1) v = v + xor_lane(v, b);
  return v;
}
template <int LPR>
__device__ __forceinline__ int lanes_sum(int v) {
#pragma unroll
  for (int b = 1; b < LPR; b <<= 1) v += xor_lane(v, b);
  return v;
}

// Root of the pairwise tree over the W (<= 16) per-wave values red[0 .. W) of a
// row: lane q < W takes value q and lanes W .. 15 exact zeros (the zero
// padding of the tree), a butterfly over lane bits 0 .. 3 pairs them in tree
// order, and lane 0's root is returned to the whole wave.
__device__ __forceinline__ float waves_tree(const float* red, int W, int lane) {
  float v = lane < W ? red[lane] : 0.0f;
#pragma unroll
  for (int b = 1; b < 16; b <<= 1) v = v + xor_lane(v, b);
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}
__device__ __forceinline__ int waves_sum(const int* red, int W, int lane) {
  int v = lane < W ? red[lane] : 0;
#pragma unroll
  for (int b = 1; b < 16; b <<= 1) v += xor_lane(v, b);
  return __builtin_amdgcn_readfirstlane(v);
}

// RELOAD: pass 2 reads each run again (from L2: the block read it moments
// before) instead of keeping the whole row in registers; used for the wide rows
// that need 8 or 16 waves per row, where 1024-thread blocks cap registers.
template <typename T, int GPW, int LPR, bool TERNARY, bool VEC, int BLOCK, bool RELOAD>
__global__ void __launch_bounds__(BLOCK)
pack_rows_kernel(const T* __restrict__ X, int64_t rows, int64_t K, int64_t sr, int64_t sk, int W,
                 int64_t row_bytes, uint8_t* __restrict__ mask, uint8_t* __restrict__ sign,
                 float* __restrict__ alpha, int32_t* __restrict__ nnz) {
  static_assert(LPR == 64 || GPW == 1, "sub-wave rows use one group");
  constexpr int NW = Raw<T>::kWords;
  constexpr int G = LPR * RUN;
  constexpr int RPW = kWave / LPR;  // rows per wave
  __shared__ float red_sum[16];
  __shared__ float red_kept[16];
  __shared__ int red_cnt[16];

  const int lane = __lane_id();
  // the wave index is wave-uniform: keep it (and what derives from it) scalar
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const int ll = lane % LPR;
  // rows handled by the block per iteration, and this lane's row among them
  const int rpb = LPR == 64 ? wpb / W : wpb * RPW;
  const int row_in_block = LPR == 64 ? wid / W : wid * RPW + lane / LPR;
  const int w_in_row = LPR == 64 ? wid - (wid / W) * W : 0;
  const float fK = (float)K;
  const int Ki = (int)K;  // K <= 65536: offsets inside a row fit 32 bits

  // wave-uniform: all GPW groups of this wave lie inside the row
  const bool full = VEC && (w_in_row * GPW + GPW) * G <= Ki;
  const int e0 = (w_in_row * GPW) * G + ll * RUN;
  // Whole-wave rows with unit stride read through a per-row buffer descriptor
  // and store the plane bytes through one: the descriptors' range checks stand
  // in for every per-lane bounds test (the row's end, padding bytes, rows past
  // the last), and the group offsets become constants.
  constexpr bool BUF = LPR == 64 && VEC;
  auto row_ptr = [&](int64_t r) { return X + (r < rows ? r : 0) * sr; };
  auto fetch_from = [&](const T* xr, int i, uint32_t (&dst)[NW]) {
    if constexpr (VEC) {
      if (full)
        load_run<T, 0>(xr, e0 + i * G, K, 1, dst);
      else
        load_run<T, 1>(xr, e0 + i * G, K, 1, dst);
    } else {
      load_run<T, 2>(xr, e0 + i * G, K, sk, dst);
    }
  };
  // Groups that lie wholly past the end of the row hold only zero padding:
  // their sums are exact zeros and they store nothing (wave-uniform).
  auto in_row_g = [&](int i) { return full || (w_in_row * GPW + i) * G < Ki; };
  auto fetch_row = [&](const T* xr, uint32_t (&dst)[GPW][NW]) {
    if (full) {
#pragma unroll
      for (int i = 0; i < GPW; ++i) load_run<T, 0>(xr, e0 + i * G, K, 1, dst[i]);
    } else {
#pragma unroll
      for (int i = 0; i < GPW; ++i) fetch_from(xr, i, dst[i]);
    }
  };
  for (int64_t r0 = (int64_t)blockIdx.x * rpb; r0 < rows; r0 += (int64_t)gridDim.x * rpb) {
    const int64_t r = r0 + row_in_block;
    const bool live = r < rows;
    const T* xrow = row_ptr(r);
    const __amdgpu_buffer_rsrc_t xs = checked_rsrc(xrow, live ? Ki * (int)sizeof(T) : 0);
    auto fetch = [&](int i, uint32_t (&dst)[NW]) {
      if constexpr (BUF)
        load_run_buf<T>(xs, e0 * (int)sizeof(T), i * G * (int)sizeof(T), dst);
      else
        fetch_from(xrow, i, dst);
    };

    uint32_t raw[RELOAD ? 1 : GPW][NW];
    if constexpr (!RELOAD) {
      if constexpr (BUF) {
#pragma unroll
        for (int i = 0; i < GPW; ++i)
          if (in_row_g(i)) fetch(i, raw[i]);
      } else {
        fetch_row(xrow, raw);
      }
    }

    auto in_row = in_row_g;

    // Pass 1: tree(|x|).
    float part[GPW];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
      part[i] = 0.0f;
      if (!in_row(i)) continue;
      if constexpr (RELOAD) fetch(i, raw[0]);
      const uint32_t* rw = raw[RELOAD ? 0 : i];
      float a[RUN];
#pragma unroll
      for (int j = 0; j < RUN; ++j) a[j] = fabsf(__uint_as_float(ebits(rw, j, T{})));
      part[i] = lane_tree<RUN>(a);
    }
    float total;
    if constexpr (LPR == 64) {
      total = wave_tree<GPW>(part);
      if (W > 1) {
        // The barriers here order LDS only: __syncthreads() would also wait for
        // every global access of the wave in flight (the previous row's plane
        // stores among them).
        if (lane == 0) red_sum[wid] = total;
        lds_barrier_local();
        total = waves_tree(&red_sum[row_in_block * W], W, lane);
        // The binary rule has no second barrier in this iteration: without this
        // one a wave could store the next row's sum over red_sum while a slower
        // wave of the same row still reads it.  (The ternary rule's second
        // barrier below already separates the two.)
        if constexpr (!TERNARY) lds_barrier_local();
      }
    } else {
      total = lanes_tree<LPR>(part[0]);
    }

    // Register pressure: make pass 2 convert the raw words again rather than
    // keep pass 1's floats alive (an empty asm that claims to change them), and
    // in RELOAD mode make it really re-read the runs (a compiler-only memory
    // barrier keeps the second loads from being merged with the first ones).
    if constexpr (RELOAD) {
      __asm__ __volatile__("" ::: "memory");
    } else {
#pragma unroll
      for (int i = 0; i < GPW; ++i)
#pragma unroll
        for (int w = 0; w < NW; ++w) __asm__ __volatile__("" : "+v"(raw[i][w]));
    }
    // Each lane stores its own byte of each plane (byte = (group*G + ll*8) / 8)
    // as soon as the group is done, so no per-group state outlives it.
    const int64_t base = (live ? r : 0) * row_bytes;
    const int boff = (w_in_row * GPW) * LPR + ll;  // this lane's byte of group 0
    const uint32_t rb = live ? (uint32_t)row_bytes : 0u;
    const __amdgpu_buffer_rsrc_t ms = checked_rsrc(TERNARY ? mask + base : sign + base, rb);
    const __amdgpu_buffer_rsrc_t ss = checked_rsrc(sign + base, rb);
    auto store_bytes = [&](int i, uint32_t mb, uint32_t sb) {
      if constexpr (BUF) {
        if constexpr (TERNARY)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)mb, ms, boff, i * LPR, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, ss, boff, i * LPR, 0);
      } else if (live && (full || boff + i * LPR < (int)row_bytes)) {
        if constexpr (TERNARY) mask[base + boff + i * LPR] = (uint8_t)mb;
        sign[base + boff + i * LPR] = (uint8_t)sb;
      }
    };
    float alpha_v;
    int count = 0;
    if constexpr (TERNARY) {
      const float mu = total / fK;
      const float thr = 0.5f * mu;
      const uint32_t uthr = __float_as_uint(thr);
      const uint32_t t2 = (uthr >> 16) * 0x10001u;  // bf16 threshold in both halves
      // Pass 2: threshold, plane bytes, tree(kept |x|), nnz.
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        part[i] = 0.0f;
        if (!in_row(i)) continue;
        if constexpr (RELOAD) fetch(i, raw[0]);
        const uint32_t* rw = raw[RELOAD ? 0 : i];
        uint32_t mb = 0, sb = 0;
        if constexpr (sizeof(T) == 2) {
          uint32_t c;
          ternary_run_bf16(raw[RELOAD ? 0 : i], t2, part[i], mb, sb, c);
          count += c;
        } else {
          float kept[RUN];
#pragma unroll
          for (int j = 0; j < RUN; ++j) {
            const uint32_t ux = ebits(rw, j, T{});
            const uint32_t ua = ux & 0x7FFFFFFFu;          // |x|
            const uint32_t keep = gt_bit(ua, uthr);        // |x| > thr
            kept[j] = __uint_as_float(ua & (0u - keep));   // keep ? |x| : +0
            mb |= keep << j;
            sb |= (keep & (ux >> 31)) << j;                // kept and negative
          }
          part[i] = lane_tree<RUN>(kept);
          count += __builtin_popcount(mb);
        }
        // Finish the group here: left alone, the compiler sinks the kept-value
        // trees past the store branches and holds every group's temporaries at
        // once (2048 x 11008 bf16: 118 VGPRs instead of 79).
        __asm__ __volatile__("" : "+v"(part[i]), "+v"(count));
        store_bytes(i, mb, sb);
      }
      float ktot;
      int ctot;
      if constexpr (LPR == 64) {
        ktot = wave_tree<GPW>(part);
        ctot = wave_sum_int(count);
        if (W > 1) {
          if (lane == 0) {
            red_kept[wid] = ktot;
            red_cnt[wid] = ctot;
          }
          lds_barrier_local();
          ktot = waves_tree(&red_kept[row_in_block * W], W, lane);
          ctot = waves_sum(&red_cnt[row_in_block * W], W, lane);
        }
      } else {
        ktot = lanes_tree<LPR>(part[0]);
        ctot = lanes_sum<LPR>(count);
      }
      count = ctot;
      alpha_v = ctot ? ktot / (float)ctot : 0.0f;
    } else {
      alpha_v = total / fK;
#pragma unroll
      for (int i = 0; i < GPW; ++i) {
        if (!in_row(i)) continue;
        if constexpr (RELOAD) fetch(i, raw[0]);
        const uint32_t* rw = raw[RELOAD ? 0 : i];
        uint32_t sb = 0;
#pragma unroll
        for (int j = 0; j < RUN; ++j) sb |= neg_bit(ebits(rw, j, T{})) << j;
        store_bytes(i, 0u, sb);
      }
    }

    if (live && w_in_row == 0 && ll == 0) {
      alpha[r] = alpha_v;
      if constexpr (TERNARY) nnz[r] = count;
    }
  }
}

// Columns of a row-major [K, C] matrix with leading dimension ld: column c
// becomes row c of the sign plane.  Block: W waves x 64 columns; wave w folds the
// aligned range [w*P/W, (w+1)*P/W) of the zero-padded length P.
constexpr int kStack = 14;  // runs per wave <= 2^13 (K <= 65536)

template <typename T, int W>
__global__ void __launch_bounds__(64 * W)
pack_columns_kernel(const T* __restrict__ X, int64_t C, int64_t K, int64_t ld, int64_t P,
                    int64_t row_bytes, uint8_t* __restrict__ sign, float* __restrict__ alpha) {
  __shared__ float red[W][64];
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  const bool live = c < C;
  const int64_t span = P / W;
  const int64_t k0 = (int64_t)wid * span;
  const int64_t runs = (span + RUN - 1) / RUN;

  float stack[kStack];
#pragma unroll
  for (int l = 0; l < kStack; ++l) stack[l] = 0.0f;
  for (int64_t n = 0; n < runs; ++n) {
    const int64_t kb = k0 + n * RUN;
    float v[RUN];
    uint32_t sb = 0;
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int64_t k = kb + j;
      float x = 0.0f;
      if (live && k < K && k < k0 + span) {
        if constexpr (sizeof(T) == 4)
          x = __uint_as_float(raw_bits(X[k * ld + c]));
        else
          x = bf16_bits_to_f32(raw_bits(X[k * ld + c]));
      }
      const uint32_t ux = __float_as_uint(x);
      v[j] = __uint_as_float(ux & 0x7FFFFFFFu);
      sb |= neg_bit(ux) << j;
    }
    float node = lane_tree<RUN>(v);
    // binary-counter merge: run n closes the levels of its trailing one bits
    bool open = true;
#pragma unroll
    for (int l = 0; l < kStack; ++l) {
      const bool merge = open && ((n >> l) & 1);
      if (merge) node = stack[l] + node;
      if (open && !merge) {
        stack[l] = node;
        open = false;
      }
    }
    if (live && kb < K) sign[c * row_bytes + kb / 8] = (uint8_t)sb;
  }
  // Root of this wave's range: pending left nodes meet zero right siblings.
  float root = 0.0f;
#pragma unroll
  for (int l = 0; l < kStack; ++l)
    if ((runs >> l) & 1) root = stack[l] + root;
  red[wid][lane] = root;
  __syncthreads();
  if (wid == 0 && live) {
    float t[W];
#pragma unroll
    for (int q = 0; q < W; ++q) t[q] = red[q][lane];
#pragma unroll
    for (int w = W; w > 1; w >>= 1)
#pragma unroll
      for (int q = 0; q < w / 2; ++q) t[q] = t[2 * q] + t[2 * q + 1];
    alpha[c] = t[0] / (float)K;
    // zero the padding bytes of the row (k in [round_up(K, 8), Kp))
    for (int64_t byte = (K + 7) / 8; byte < row_bytes; ++byte) sign[c * row_bytes + byte] = 0;
  }
}

// Staged column kernel (fast path: 16-byte aligned rows, C a multiple of the
// 16-byte vector, padded length P >= 16 S).  A block of 16 waves packs 64
// columns.  Wave w owns the aligned range [w P/16, (w+1) P/16) of the padded
// length, cut into segments of S rows (S = 32 for bf16, 16 for fp32); in chunk
// q the block loads segment q of all 16 ranges (16 S rows x 64 columns, 64 KiB)
// with 16-byte loads into LDS, and lane c of wave w reads its column of its
// segment from there: the segment is an aligned sub-tree, folded into the
// wave's binary-counter stack like the runs above, and its S sign bits are S/8
// whole bytes of the plane.  The next chunk's loads are in flight while the
// current one is reduced.
template <typename T>
struct ColStage {
  static constexpr int S = sizeof(T) == 2 ? 32 : 16;  // rows per segment
  static constexpr int VPR = 64 * (int)sizeof(T) / 16;  // 16-byte vectors per tile row
  static constexpr int UNITS = 16 * S * VPR / 1024;      // vectors per thread per chunk
};

template <typename T>
__global__ void __launch_bounds__(1024)
pack_columns_staged_kernel(const T* __restrict__ X, int64_t C, int64_t K, int64_t ld, int64_t P,
                           int64_t row_bytes, uint8_t* __restrict__ sign,
                           float* __restrict__ alpha) {
  constexpr int S = ColStage<T>::S, VPR = ColStage<T>::VPR, UNITS = ColStage<T>::UNITS;
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per vector
  __shared__ __attribute__((aligned(16))) T tile[16 * S][64];
  __shared__ float red[16][64];
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t c = c0 + lane;
  const bool live = c < C;
  const int64_t span = P / 16;
  const int64_t nchunks = span / S;

  auto fetch = [&](int64_t q, u32x4 (&buf)[UNITS]) {
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = i * 1024 + (int)threadIdx.x;
      const int rr = u / VPR, v = u % VPR;
      const int64_t k = (int64_t)(rr / S) * span + q * S + rr % S;
      const int64_t col = c0 + (int64_t)v * EPV;
      buf[i] = (k < K && col < C) ? *reinterpret_cast<const u32x4*>(X + k * ld + col)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 buf[UNITS];
  fetch(0, buf);

  float stack[kStack];
#pragma unroll
  for (int l = 0; l < kStack; ++l) stack[l] = 0.0f;
  for (int64_t q = 0; q < nchunks; ++q) {
    lds_barrier_local();  // the previous chunk's tile has been read
#pragma unroll
    for (int i = 0; i < UNITS; ++i) {
      const int u = i * 1024 + (int)threadIdx.x;
      *reinterpret_cast<u32x4*>(&tile[u / VPR][(u % VPR) * EPV]) = buf[i];
    }
    if (q + 1 < nchunks) fetch(q + 1, buf);
    lds_barrier_local();
    float v[S];
    uint32_t sb = 0;
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const uint32_t ux = sizeof(T) == 4 ? raw_bits(tile[wid * S + j][lane])
                                         : raw_bits(tile[wid * S + j][lane]) << 16;
      v[j] = __uint_as_float(ux & 0x7FFFFFFFu);
      sb |= neg_bit(ux) << j;
    }
    float node = lane_tree<S>(v);
    bool open = true;
#pragma unroll
    for (int l = 0; l < kStack; ++l) {
      const bool merge = open && ((q >> l) & 1);
      if (merge) node = stack[l] + node;
      if (open && !merge) {
        stack[l] = node;
        open = false;
      }
    }
    const int64_t b0 = ((int64_t)wid * span + q * S) / 8;  // first plane byte of the segment
    if (live && b0 < row_bytes) {
      if constexpr (S == 32)
        *reinterpret_cast<uint32_t*>(sign + c * row_bytes + b0) = sb;
      else
        *reinterpret_cast<uint16_t*>(sign + c * row_bytes + b0) = (uint16_t)sb;
    }
  }
  float root = 0.0f;
#pragma unroll
  for (int l = 0; l < kStack; ++l)
    if ((nchunks >> l) & 1) root = stack[l] + root;
  red[wid][lane] = root;
  __syncthreads();
  if (wid == 0 && live) {
    float t[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) t[q] = red[q][lane];
    alpha[c] = lane_tree<16>(t) / (float)K;
  }
}

// Two-plane residual binarization (BiLLM page, Approach: residual binarization
// of salient weights; here whole rows): plane 1 and alpha1 as the binary rule,
// plane 2 and alpha2 the binary rule on r = w - alpha1 * s1 (fp32; the padding
// stays zero).  One wave per row, four rows per block; lane l owns the aligned
// range [l E, (l+1) E) of the row padded to 64 E >= max(P, 512) values (zeros
// past P leave the root unchanged), folds its runs of 8 into a binary-counter
// stack, and the 64 lane roots meet in a butterfly (lane bit 0 first), so both
// sums follow the pairwise tree exactly.  Output rows are interleaved in groups
// of 32: weight row n -> plane row 64 (n / 32) + n % 32 (plane 1), that + 32
// (plane 2); alpha likewise.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256)
pack_residual_kernel(const T* __restrict__ X, int64_t rows, int64_t K, int64_t sr, int64_t E,
                     int64_t row_bytes, uint8_t* __restrict__ sign, float* __restrict__ alpha) {
  const int lane = __lane_id();
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= rows) return;  // whole waves leave together; no block barrier below
  const T* xrow = X + r * sr;
  const int64_t out1 = 64 * (r >> 5) + (r & 31), out2 = out1 + 32;
  const int64_t runs = E / RUN;
  const int64_t e_lane = (int64_t)lane * E;
  constexpr int NW = Raw<T>::kWords;
  auto fetch = [&](int64_t e, uint32_t (&raw)[NW]) {
    if constexpr (VEC)
      load_run<T, 1>(xrow, e, K, 1, raw);
    else
      load_run<T, 2>(xrow, e, K, 1, raw);
  };
  float a1 = 0.0f;
#pragma unroll 1
  for (int plane = 0; plane < 2; ++plane) {
    float stack[kStack];
#pragma unroll
    for (int l = 0; l < kStack; ++l) stack[l] = 0.0f;
    uint8_t* srow = sign + (plane ? out2 : out1) * row_bytes;
#pragma unroll 1
    for (int64_t n = 0; n < runs; ++n) {
      const int64_t e = e_lane + n * RUN;
      uint32_t raw[NW];
      fetch(e, raw);
      float v[RUN];
      uint32_t sb = 0;
#pragma unroll
      for (int j = 0; j < RUN; ++j) {
        uint32_t ux = ebits(raw, j, T{});
        if (plane == 1 && e + j < K) {
          const float x = __uint_as_float(ux);
          ux = __float_as_uint(neg_bit(ux) ? x + a1 : x - a1);
        }
        v[j] = __uint_as_float(ux & 0x7FFFFFFFu);
        sb |= neg_bit(ux) << j;
      }
      float node = lane_tree<RUN>(v);
      bool open = true;
#pragma unroll
      for (int l = 0; l < kStack; ++l) {
        const bool merge = open && ((n >> l) & 1);
        if (merge) node = stack[l] + node;
        if (open && !merge) {
          stack[l] = node;
          open = false;
        }
      }
      const int64_t byte = e / 8;
      if (byte < row_bytes) srow[byte] = (uint8_t)sb;
    }
    float root = 0.0f;
#pragma unroll
    for (int l = 0; l < kStack; ++l)
      if ((runs >> l) & 1) root = stack[l] + root;
#pragma unroll
    for (int b = 0; b < 6; ++b) root = root + __shfl_xor(root, 1 << b, kWave);
    const float al = root / (float)K;
    if (plane == 0) a1 = al;
    if (lane == 0) alpha[plane ? out2 : out1] = al;
  }
}

template <typename T>
hipError_t launch_residual(const T* X, int64_t rows, int64_t K, int64_t sr, uint8_t* sign,
                           float* alpha, hipStream_t stream) {
  int64_t P = 1;
  while (P < K) P <<= 1;
  const int64_t E = P / 64 > RUN ? P / 64 : RUN;
  const int64_t row_bytes = (K + 63) / 64 * 8;
  const bool vec = K % RUN == 0 && reinterpret_cast<uintptr_t>(X) % 16 == 0 &&
                   (sr * (int64_t)sizeof(T)) % 16 == 0;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (vec)
    hipLaunchKernelGGL((pack_residual_kernel<T, true>), grid, dim3(256), 0, stream, X, rows, K, sr,
                       E, row_bytes, sign, alpha);
  else
    hipLaunchKernelGGL((pack_residual_kernel<T, false>), grid, dim3(256), 0, stream, X, rows, K,
                       sr, E, row_bytes, sign, alpha);
  return hipGetLastError();
}

struct Plan {
  int lpr;    // lanes per row (16, 32 or 64)
  int gpw;    // groups per wave
  int W;      // waves per row: those that hold data.  The tree runs over the
              // power of two above W; the missing waves' sums are exact zeros,
              // which the zero-padded LDS tree supplies.
  int block;  // threads per block (a multiple of 64 * W)
  int bound;  // the kernel's launch bound (256, 512 or 1024)
};

// Rows up to 4096 values: one wave per row (8 groups of 512 at most) and four
// rows per block.  Up to 16384 values: 8 groups per wave and as many waves per
// row as hold data (11008: 3 waves, the last one partly padding, whose empty
// groups are skipped), in blocks of at most 256 threads.  Up to 32768 values:
// 4 groups per wave, up to 16 waves per row in blocks of 1024 threads.  Beyond:
// 8 groups per wave that re-read their runs in pass 2.
Plan plan_for(int64_t K) {
  Plan pl;
  if (K <= 16 * RUN) return {16, 1, 1, 256, 256};
  if (K <= 32 * RUN) return {32, 1, 1, 256, 256};
  const int64_t n = (K + 64 * RUN - 1) / (64 * RUN);  // groups holding data
  int64_t p = 1;
  while (p < n) p <<= 1;
  pl.lpr = 64;
  if (p <= 8) {
    pl.gpw = (int)p;
    pl.W = 1;
    pl.block = pl.bound = 256;
  } else if (p <= 32) {
    pl.gpw = 8;
    pl.bound = 256;
  } else if (p <= 64) {
    pl.gpw = 4;
    pl.bound = 1024;
  } else {
    pl.gpw = 8;
    pl.bound = 1024;
  }
  pl.W = (int)((n + pl.gpw - 1) / pl.gpw);
  pl.block = (pl.bound / kWave / pl.W) * pl.W * kWave;  // whole rows per block
  return pl;
}

template <typename T, bool TERNARY, bool VEC>
hipError_t launch_rows(const T* X, int64_t rows, int64_t K, int64_t sr, int64_t sk, uint8_t* mask,
                       uint8_t* sign, float* alpha, int32_t* nnz, hipStream_t stream) {
  const Plan pl = plan_for(K);
  const int64_t row_bytes = (K + 63) / 64 * 8;
  const int wpb = pl.block / kWave;
  const int rpb = pl.lpr == 64 ? wpb / pl.W : wpb * (kWave / pl.lpr);
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  const dim3 grid((unsigned)blocks), block((unsigned)pl.block);
#define BWTA_ROWS(GPW_, LPR_, BLOCK_, RELOAD_)                                                  \
  hipLaunchKernelGGL((pack_rows_kernel<T, GPW_, LPR_, TERNARY, VEC, BLOCK_, RELOAD_>), grid,      \
                     block, 0, stream, X, rows, K, sr, sk, pl.W, row_bytes, mask, sign, alpha, nnz)
  if (pl.lpr == 16) {
    BWTA_ROWS(1, 16, 256, false);
  } else if (pl.lpr == 32) {
    BWTA_ROWS(1, 32, 256, false);
  } else if (pl.W == 1) {
    switch (pl.gpw) {
      case 1: BWTA_ROWS(1, 64, 256, false); break;
      case 2: BWTA_ROWS(2, 64, 256, false); break;
      case 4: BWTA_ROWS(4, 64, 256, false); break;
      default: BWTA_ROWS(8, 64, 256, false); break;
    }
  } else if (pl.gpw == 8 && pl.bound == 256) {
    BWTA_ROWS(8, 64, 256, false);
  } else if (pl.gpw == 4) {
    BWTA_ROWS(4, 64, 1024, false);
  } else {
    BWTA_ROWS(8, 64, 1024, true);
  }
#undef BWTA_ROWS
  return hipGetLastError();
}

template <typename T>
hipError_t launch_columns(const T* X, int64_t C, int64_t K, int64_t ld, uint8_t* sign,
                          float* alpha, hipStream_t stream) {
  int64_t P = 1;
  while (P < K) P <<= 1;
  const int64_t row_bytes = (K + 63) / 64 * 8;
  const dim3 grid((unsigned)((C + 63) / 64));
  constexpr int EPV = 16 / (int)sizeof(T);
  if (P >= 16 * ColStage<T>::S && C % EPV == 0 && ld % EPV == 0 &&
      reinterpret_cast<uintptr_t>(X) % 16 == 0 && row_bytes % 4 == 0) {
    hipLaunchKernelGGL((pack_columns_staged_kernel<T>), grid, dim3(1024), 0, stream, X, C, K, ld,
                       P, row_bytes, sign, alpha);
    return hipGetLastError();
  }
  // W waves split the padded length P; each range must hold whole runs of 8.
  if (P >= 16 * RUN) {
    hipLaunchKernelGGL((pack_columns_kernel<T, 16>), grid, dim3(1024), 0, stream, X, C, K, ld, P,
                       row_bytes, sign, alpha);
  } else if (P >= 4 * RUN) {
    hipLaunchKernelGGL((pack_columns_kernel<T, 4>), grid, dim3(256), 0, stream, X, C, K, ld, P,
                       row_bytes, sign, alpha);
  } else {
    hipLaunchKernelGGL((pack_columns_kernel<T, 1>), grid, dim3(64), 0, stream, X, C, K, ld, P,
                       row_bytes, sign, alpha);
  }
  return hipGetLastError();
}

template <bool TERNARY>
hipError_t launch_any(const void* X, Elt dt, int64_t rows, int64_t K, int64_t sr, int64_t sk,
                      uint8_t* mask, uint8_t* sign, float* alpha, int32_t* nnz, hipStream_t stream) {
  const size_t es = dt == Elt::F32 ? 4 : 2;
  if (!TERNARY && sk != 1 && sr == 1 && sk >= rows) {
    return dt == Elt::F32
               ? launch_columns<float>(static_cast<const float*>(X), rows, K, sk, sign, alpha, stream)
               : launch_columns<uint16_t>(static_cast<const uint16_t*>(X), rows, K, sk, sign, alpha,
                                          stream);
  }
  const bool vec = sk == 1 && K % RUN == 0 && (reinterpret_cast<uintptr_t>(X) % 16 == 0) &&
                   ((sr * (int64_t)es) % 16 == 0 || rows <= 1);
  if (dt == Elt::F32) {
    auto p = static_cast<const float*>(X);
    return vec ? launch_rows<float, TERNARY, true>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream)
               : launch_rows<float, TERNARY, false>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream);
  }
  auto p = static_cast<const uint16_t*>(X);
  return vec ? launch_rows<uint16_t, TERNARY, true>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream)
             : launch_rows<uint16_t, TERNARY, false>(p, rows, K, sr, sk, mask, sign, alpha, nnz, stream);
}

}  // namespace

hipError_t launch_ternarize(const void* X, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                            uint8_t* mask, uint8_t* sign, float* alpha, int32_t* nnz,
                            hipStream_t stream) {
  return launch_any<true>(X, dt, rows, K, stride_row, 1, mask, sign, alpha, nnz, stream);
}

hipError_t launch_binarize_residual(const void* W, Elt dt, int64_t rows, int64_t K,
                                   int64_t stride_row, uint8_t* sign, float* alpha,
                                   hipStream_t stream) {
  return dt == Elt::F32 ? launch_residual<float>(static_cast<const float*>(W), rows, K, stride_row,
                                                 sign, alpha, stream)
                        : launch_residual<uint16_t>(static_cast<const uint16_t*>(W), rows, K,
                                                    stride_row, sign, alpha, stream);
}

hipError_t launch_binarize(const void* W, Elt dt, int64_t rows, int64_t K, int64_t stride_row,
                           int64_t stride_k, uint8_t* sign, float* alpha, hipStream_t stream) {
  return launch_any<false>(W, dt, rows, K, stride_row, stride_k, nullptr, sign, alpha, nullptr,
                           stream);
}

}  // namespace bwta
