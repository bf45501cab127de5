// gemm_popcount.hip - the same binary x ternary products on the vector ALUs
// with population counts, and the decode GEMV.
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: bit-packed binary/ternary MatMul.
// With t = mask * (1 - 2 sign_a) and s = 1 - 2 w, t*s = mask * (1 - 2 (sign_a ^ w)),
// so for one 32-bit word
//   sum t*s = popc(mask) - 2 popc(mask & (sign_a ^ w))
//           = popc(mask) - 2 popc(bfi(w, mask ^ sign_a, sign_a))
// (sign_a is a subset of mask), i.e. one v_bfi_b32 and one accumulating
// v_bcnt_u32_b32 per 32 products, and acc = nnz - 2 * sum_words popc(...).
// For ternary x ternary (attention Q K^T):
//   sum tq*tk = popc(mq & mk) - 2 popc(mq & mk & (aq ^ ak)).
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

template <int OUT>
__device__ __forceinline__ void store_out(void* Y, int64_t idx, int acc, float sa, float sb) {
  if constexpr (OUT == (int)Elt::I32) {
    reinterpret_cast<int32_t*>(Y)[idx] = acc;
  } else {
    const float sc = sa * sb;
    const float y = (float)acc * sc;
    if constexpr (OUT == (int)Elt::F32)
      reinterpret_cast<float*>(Y)[idx] = y;
    else
      reinterpret_cast<uint16_t*>(Y)[idx] = f32_to_bf16_rne(y);
  }
}

// ---------------------------------------------------------------------------
// GEMM: block tile 64 (M) x 128 (N), 256 threads, each thread 4 x 8 outputs.
// k advances in chunks of 16 words (512 k) staged in LDS.  A is staged as
// (mask ^ sign, sign), B as sign (binary) or (mask, sign) (ternary).
// ---------------------------------------------------------------------------
constexpr int PBM = 64, PBN = 128, PKC = 16;  // tile rows, tile cols, words per chunk
constexpr int PLD = PKC + 4;                  // padded LDS row length in words

template <bool B_TERNARY, int OUT>
__global__ void __launch_bounds__(256)
gemm_popcount_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                     const float* __restrict__ a_alpha, const int32_t* __restrict__ a_nnz,
                     int64_t a_batch_rows, const uint8_t* __restrict__ b_mask,
                     const uint8_t* __restrict__ b_sign, const float* __restrict__ b_alpha,
                     int64_t b_batch_rows, int64_t M, int64_t N, int64_t row_bytes, int tiles_n,
                     void* __restrict__ Y, int64_t ldy, int64_t y_batch_stride) {
  __shared__ uint32_t sa_p[PBM * PLD], sa_s[PBM * PLD];
  __shared__ uint32_t sb_s[PBN * PLD];
  __shared__ uint32_t sb_m[B_TERNARY ? PBN * PLD : 1];

  const int tid = threadIdx.x;
  const int tn = tid & 15, tm = tid >> 4;
  const int64_t b = blockIdx.z;
  const int tile_m = blockIdx.x / tiles_n;
  const int tile_n = blockIdx.x - tile_m * tiles_n;
  const int64_t m0 = (int64_t)tile_m * PBM, n0 = (int64_t)tile_n * PBN;
  const int64_t a_row0 = b * a_batch_rows + m0, b_row0 = b * b_batch_rows + n0;
  const int64_t words = row_bytes / 4;
  const uint32_t* A_m = reinterpret_cast<const uint32_t*>(a_mask + a_row0 * row_bytes);
  const uint32_t* A_s = reinterpret_cast<const uint32_t*>(a_sign + a_row0 * row_bytes);
  const uint32_t* B_s = reinterpret_cast<const uint32_t*>(b_sign + b_row0 * row_bytes);
  const uint32_t* B_m =
      B_TERNARY ? reinterpret_cast<const uint32_t*>(b_mask + b_row0 * row_bytes) : nullptr;
  const int64_t w_stride = row_bytes / 4;

  int pos[4][8], neg[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) pos[i][j] = neg[i][j] = 0;

  for (int64_t k0 = 0; k0 < words; k0 += PKC) {
    // Stage: A 64 rows x 16 words (4 per thread), B 128 rows x 16 words (8 per thread).
    for (int e = tid; e < PBM * PKC; e += 256) {
      const int row = e / PKC, w = e - row * PKC;
      const bool ok = m0 + row < M && k0 + w < words;
      const uint32_t mm = ok ? A_m[row * w_stride + k0 + w] : 0u;
      const uint32_t ss = ok ? A_s[row * w_stride + k0 + w] : 0u;
      sa_p[row * PLD + w] = B_TERNARY ? mm : (mm ^ ss);
      sa_s[row * PLD + w] = ss;
    }
    for (int e = tid; e < PBN * PKC; e += 256) {
      const int row = e / PKC, w = e - row * PKC;
      const bool ok = n0 + row < N && k0 + w < words;
      sb_s[row * PLD + w] = ok ? B_s[row * w_stride + k0 + w] : 0u;
      if constexpr (B_TERNARY) sb_m[row * PLD + w] = ok ? B_m[row * w_stride + k0 + w] : 0u;
    }
    __syncthreads();
#pragma unroll 1
    for (int w0 = 0; w0 < PKC; w0 += 4) {
      uint4 ap[4], as[4], bs[8], bm[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ap[i] = *reinterpret_cast<const uint4*>(&sa_p[(4 * tm + i) * PLD + w0]);
        as[i] = *reinterpret_cast<const uint4*>(&sa_s[(4 * tm + i) * PLD + w0]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bs[j] = *reinterpret_cast<const uint4*>(&sb_s[(tn + 16 * j) * PLD + w0]);
        if constexpr (B_TERNARY) bm[j] = *reinterpret_cast<const uint4*>(&sb_m[(tn + 16 * j) * PLD + w0]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t pa[4] = {ap[i].x, ap[i].y, ap[i].z, ap[i].w};
          const uint32_t sa[4] = {as[i].x, as[i].y, as[i].z, as[i].w};
          const uint32_t sw[4] = {bs[j].x, bs[j].y, bs[j].z, bs[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (B_TERNARY) {
              const uint32_t mw[4] = {bm[j].x, bm[j].y, bm[j].z, bm[j].w};
              const uint32_t both = pa[q] & mw[q];  // pa holds the A mask here
              pos[i][j] += __builtin_popcount(both);
              neg[i][j] += __builtin_popcount(both & (sa[q] ^ sw[q]));
            } else {
              neg[i][j] += __builtin_popcount((sw[q] & pa[q]) | (~sw[q] & sa[q]));
            }
          }
        }
    }
    __syncthreads();
  }

  // Epilogue.  Thread (tm, tn) owns rows 4 tm + i and columns tn + 16 j.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 4 * tm + i;
    if (m >= M) continue;
    const int nz = B_TERNARY ? 0 : a_nnz[b * a_batch_rows + m];
    const float sa = OUT == (int)Elt::I32 ? 0.0f : a_alpha[b * a_batch_rows + m];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = n0 + tn + 16 * j;
      if (n >= N) continue;
      const int acc = B_TERNARY ? pos[i][j] - 2 * neg[i][j] : nz - 2 * neg[i][j];
      const float sb = OUT == (int)Elt::I32 ? 0.0f : b_alpha[b * b_batch_rows + n];
      store_out<OUT>(Y, b * y_batch_stride + m * ldy + n, acc, sa, sb);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMV (M <= 16): one wave streams whole weight rows; lane l covers bytes
// [16 l + 1024 c, +16) of every row for chunks c < NCH, so each wave-wide load
// is one contiguous 1 KiB run, and the activation words it meets are the same
// for every row: they stay in registers.  MB activation rows are handled per
// pass.  R rows are accumulated per lane before one reduce-scatter across the
// wave (integer sums, exact in any order).
// ---------------------------------------------------------------------------
template <int V>
__device__ __forceinline__ void wave_reduce_scatter_int(int (&v)[V]) {
  // After this, lane l holds in v[0] the wave total of value index bitrev(l mod V).
  const int lane = __lane_id();
  int s = 0;
#pragma unroll
  for (int cnt = V; cnt > 1; cnt >>= 1, ++s) {
    const bool hi = (lane >> s) & 1;
#pragma unroll
    for (int j = 0; j < cnt / 2; ++j) {
      const int keep = hi ? v[j + cnt / 2] : v[j];
      const int send = hi ? v[j] : v[j + cnt / 2];
      v[j] = keep + __shfl_xor(send, 1 << s, kWave);
    }
  }
#pragma unroll
  for (int b = s; b < 6; ++b) v[0] += __shfl_xor(v[0], 1 << b, kWave);
}

template <int BITS>
__device__ __forceinline__ int bitrev(int x) {
  int r = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) r |= ((x >> i) & 1) << (BITS - 1 - i);
  return r;
}

// RES: two-plane residual weights, planes interleaved in groups of 32 rows; N
// counts outputs.  A wave takes two adjacent outputs o, o + 1 (o even) and
// their four plane rows b, b + 1 (plane 1) and b + 32, b + 33 (plane 2),
// b = 64 (o / 32) + o % 32, and each output lane fetches its plane-2 count from
// the lane that holds it: y = acc1 * (alpha_a * alpha1) + acc2 * (alpha_a * alpha2).
template <int MB, int NCH, int R, int OUT, bool RES = false>
__global__ void __launch_bounds__(256)
gemv_popcount_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                     const float* __restrict__ a_alpha, const int32_t* __restrict__ a_nnz,
                     int m_base, int m_count, const uint8_t* __restrict__ w_sign,
                     const float* __restrict__ w_alpha, int64_t N, int64_t row_bytes,
                     void* __restrict__ Y, int64_t ldy) {
  constexpr int V = R * MB;
  constexpr int LOGV = V == 1 ? 0 : V == 2 ? 1 : V == 4 ? 2 : V == 8 ? 3 : V == 16 ? 4 : 5;
  static_assert((1 << LOGV) == V, "R * MB must be a power of two <= 32");
  const int lane = __lane_id();
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;

  // Activation words of this lane's chunks: p = mask ^ sign, s = sign.
  uint32_t ap[MB][NCH][4], as[MB][NCH][4];
  bool cvalid[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t off = (int64_t)c * 1024 + lane * 16;
    cvalid[c] = off < row_bytes;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const bool ok = cvalid[c] && m < m_count;
      const int64_t row = m_base + (m < m_count ? m : 0);
      uint4 mm = ok ? *reinterpret_cast<const uint4*>(a_mask + row * row_bytes + off) : uint4{0, 0, 0, 0};
      uint4 ss = ok ? *reinterpret_cast<const uint4*>(a_sign + row * row_bytes + off) : uint4{0, 0, 0, 0};
      ap[m][c][0] = mm.x ^ ss.x; ap[m][c][1] = mm.y ^ ss.y;
      ap[m][c][2] = mm.z ^ ss.z; ap[m][c][3] = mm.w ^ ss.w;
      as[m][c][0] = ss.x; as[m][c][1] = ss.y; as[m][c][2] = ss.z; as[m][c][3] = ss.w;
    }
  }
  int nz[MB];
  float sa[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int64_t row = m_base + (m < m_count ? m : 0);
    nz[m] = a_nnz[row];
    sa[m] = OUT == (int)Elt::I32 ? 0.0f : a_alpha[row];
  }

  static_assert(!RES || (R == 4 && OUT != (int)Elt::I32), "two-plane rows come in fours");
  constexpr int STEP = RES ? 2 : R;  // outputs per wave iteration
  for (int64_t n0 = wave * STEP; n0 < N; n0 += nwaves * STEP) {
    int cnt[V];
#pragma unroll
    for (int i = 0; i < V; ++i) cnt[i] = 0;
    const int64_t pbase = 64 * (n0 >> 5) + (n0 & 31);  // RES: plane row of output n0
    u32x4 w[R][NCH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int64_t n = RES ? pbase + (r & 1) + (r >> 1) * 32 : (n0 + r < N ? n0 + r : N - 1);
        w[r][c] = cvalid[c] ? load_nt16(w_sign + n * row_bytes + (int64_t)c * 1024 + lane * 16)
                            : u32x4{0, 0, 0, 0};
      }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t ww[4] = {w[r][c].x, w[r][c].y, w[r][c].z, w[r][c].w};
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cnt[r * MB + m] += __builtin_popcount((ww[q] & ap[m][c][q]) | (~ww[q] & as[m][c][q]));
      }
    wave_reduce_scatter_int<V>(cnt);
    if constexpr (RES) {
      const int v = bitrev<LOGV>(lane & (V - 1));
      const int other = __shfl(cnt[0], bitrev<LOGV>(v ^ (2 * MB)), kWave);  // plane 2
      const int r = v / MB, m = v - r * MB;
      if (lane < V && r < 2 && m < m_count) {
        float sam = sa[0];
#pragma unroll
        for (int mm = 1; mm < MB; ++mm) sam = m == mm ? sa[mm] : sam;
        int nzm = nz[0];
#pragma unroll
        for (int mm = 1; mm < MB; ++mm) nzm = m == mm ? nz[mm] : nzm;
        const float a1 = w_alpha[pbase + r], a2 = w_alpha[pbase + r + 32];
        const float y1 = (float)(nzm - 2 * cnt[0]) * (sam * a1);
        const float y2 = (float)(nzm - 2 * other) * (sam * a2);
        const float y = y1 + y2;
        const int64_t idx = (int64_t)(m_base + m) * ldy + n0 + r;
        if constexpr (OUT == (int)Elt::F32)
          reinterpret_cast<float*>(Y)[idx] = y;
        else
          reinterpret_cast<uint16_t*>(Y)[idx] = f32_to_bf16_rne(y);
      }
      continue;
    }
    if (lane < V) {
      const int v = bitrev<LOGV>(lane);
      const int r = v / MB, m = v - r * MB;
      const int64_t n = n0 + r;
      if (n < N && m < m_count) {
        const float sb = OUT == (int)Elt::I32 ? 0.0f : w_alpha[n];
        // select sa[m] without dynamic register indexing
        float sam = sa[0];
#pragma unroll
        for (int mm = 1; mm < MB; ++mm) sam = m == mm ? sa[mm] : sam;
        int nzm = nz[0];
#pragma unroll
        for (int mm = 1; mm < MB; ++mm) nzm = m == mm ? nz[mm] : nzm;
        store_out<OUT>(Y, (int64_t)(m_base + m) * ldy + n, nzm - 2 * cnt[0], sam, sb);
      }
    }
  }
}

// Decode linear of ONE activation row in one launch (bwta_gemv_fused, M = 1):
// every block ternarizes the row itself into LDS planes, then its waves stream
// weight rows exactly as gemv_popcount_kernel does.  Each thread loads its share
// of the row first; the wave's first weight loads go out as soon as that share
// is in, so the rest of the ternarization runs under them.  Every block repeats
// the ternarization, so blocks are as wide as the grid allows (WB = 4, 8 or 16
// waves): the repeated work scales with the number of blocks.
//
// The block's ternarization follows the definition's tree: thread t < NT owns
// the aligned range [t V, t V + V) of the row zero-padded to P = 2^ceil(log2 K)
// (NT = min(64 WB, P / 8), V = P / NT), sums its runs of 8 in a pairwise tree,
// and the 64 WB thread sums (zeros past NT) meet in a butterfly over the lanes
// and a tree over the WB waves - all aligned sub-trees of the row's tree, so
// mu, thr, the kept-value tree, nnz and alpha_a equal bwta_ternarize_pack's bit
// for bit.  The row stays in registers between the two passes; pass 2 writes
// the plane bytes into LDS.
constexpr int kFusedMaxK = 32768;  // runs per thread <= 16 (bf16; fp32 rows up to 16384: <= 8)
constexpr int kFusedPlaneBytes = kFusedMaxK / 8;
constexpr int64_t kFusedRowWaves = 8192;  // grid cap (32 waves per compute unit)
constexpr int64_t kFusedCUs = 256;

template <typename TX>
struct RowRun {
  static constexpr int kWords = 8 * (int)sizeof(TX) / 4;  // 32-bit words per run of 8
};

// Raw words of the run at byte offset `off` of the row (K a multiple of 8: a run
// is wholly in or out of the row; out of range, or off < 0, reads zeros).
// Buffer loads with no branch around them, so the wait for the row's runs does
// not also wait for the weight loads issued after them.
template <typename TX>
__device__ __forceinline__ void load_row_run(__amdgpu_buffer_rsrc_t xrs, int off,
                                             uint32_t (&w)[RowRun<TX>::kWords]) {
  constexpr int NW = RowRun<TX>::kWords;
  const int o = off < 0 ? 0x40000000 : off;
#pragma unroll
  for (int v = 0; v < NW / 4; ++v) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(xrs, o + 16 * v, 0, 0);
    w[4 * v + 0] = u.x;
    w[4 * v + 1] = u.y;
    w[4 * v + 2] = u.z;
    w[4 * v + 3] = u.w;
  }
}

template <typename TX>
__device__ __forceinline__ void row_run_values(const uint32_t (&w)[RowRun<TX>::kWords], float (&v)[8]) {
  if constexpr (sizeof(TX) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(w[j]);
  }
}

// Root of the block's tree over its WB waves' threads' values (thread order).
template <int WB>
__device__ __forceinline__ float block_tree(float v, float* red) {
  const int lane = __lane_id(), wid = threadIdx.x / kWave;
#pragma unroll
  for (int b = 0; b < 6; ++b) v = v + xor_lane(v, 1 << b);
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float w[WB];
#pragma unroll
  for (int i = 0; i < WB; ++i) w[i] = red[i];
  __syncthreads();
  return lane_tree<WB>(w);
}
template <int WB>
__device__ __forceinline__ int block_sum(int v, int* ired) {
  const int lane = __lane_id(), wid = threadIdx.x / kWave;
#pragma unroll
  for (int b = 0; b < 6; ++b) v += xor_lane(v, 1 << b);
  if (lane == 0) ired[wid] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < WB; ++i) r += ired[i];
  __syncthreads();
  return r;
}

template <int NCH, typename TX, int OUT, int RUNS, int WB>
__global__ void __launch_bounds__(WB * 64)
gemv_fused_row_kernel(const TX* __restrict__ X, int K, const uint8_t* __restrict__ w_sign,
                      const float* __restrict__ w_alpha, int64_t N, int64_t row_bytes,
                      void* __restrict__ Y, uint8_t* __restrict__ o_mask,
                      uint8_t* __restrict__ o_sign, float* __restrict__ o_alpha,
                      int32_t* __restrict__ o_nnz) {
  constexpr int R = 4;  // weight rows per wave and iteration, as in gemv_popcount_kernel
  __shared__ __attribute__((aligned(16))) uint8_t s_mask[kFusedPlaneBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_sign[kFusedPlaneBytes];
  __shared__ float red[WB];
  __shared__ int ired[WB];
  const int lane = __lane_id();
  const int t = threadIdx.x;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + t) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;

  // 1. the row's runs of this thread (RUNS >= its runs)
  constexpr int NWR = RowRun<TX>::kWords;
  int P = 8;
  while (P < K) P <<= 1;
  const int NT = P / 8 < WB * kWave ? P / 8 : WB * kWave;
  const int V = P / NT;
  const int runs = V / 8;  // a power of two <= RUNS
  const bool part = t < NT;
  const __amdgpu_buffer_rsrc_t xrs = checked_rsrc(X, (uint32_t)K * (uint32_t)sizeof(TX));
  uint32_t xr[RUNS][NWR];
#pragma unroll
  for (int r = 0; r < RUNS; ++r)
    load_row_run<TX>(xrs, part && r < runs ? (t * V + 8 * r) * (int)sizeof(TX) : -1, xr[r]);
  // A lane's chunk past the row end loads the row's first bytes instead: its
  // activation words are zero there, so those weight bits count nothing.
  bool cvalid[NCH];
  int64_t coff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    cvalid[c] = (int64_t)c * 1024 + lane * 16 < row_bytes;
    coff[c] = cvalid[c] ? (int64_t)c * 1024 + lane * 16 : 0;
  }
  u32x4 w[R][NCH];
  auto load_w = [&](int64_t n0) {  // rows past N re-read row N - 1; nothing stores them
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int64_t n = n0 + r < N ? n0 + r : N - 1;
        w[r][c] = load_nt16(w_sign + n * row_bytes + coff[c]);
      }
  };

  // 2. ternarize the row into the LDS planes; the weight loads go out once the
  // row's runs are in (issued earlier, they would queue ahead of other waves' row
  // reads and hold up every block's ternarization)
  float rs[RUNS];
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {  // runs past `runs` hold zeros: exact zero sums
    float v[8];
    row_run_values<TX>(xr[r], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fabsf(v[j]);
    rs[r] = lane_tree<8>(v);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_w(wave * R);
  for (int i = t; i < (int)(row_bytes / 4); i += blockDim.x) {
    reinterpret_cast<uint32_t*>(s_mask)[i] = 0u;
    reinterpret_cast<uint32_t*>(s_sign)[i] = 0u;
  }
  const float total = block_tree<WB>(lane_tree<RUNS>(rs), red);
  const float thr = 0.5f * (total / (float)K);
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < RUNS; ++r) {
    rs[r] = 0.0f;
    if (part && r < runs) {
      float v[8], kept[8];
      row_run_values<TX>(xr[r], v);
      uint32_t mb = 0, sb = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = fabsf(v[j]);
        const bool keep = a > thr;
        kept[j] = keep ? a : 0.0f;
        mb |= (uint32_t)keep << j;
        sb |= (uint32_t)(keep && v[j] < 0.0f) << j;
      }
      rs[r] = lane_tree<8>(kept);
      cnt += __builtin_popcount(mb);
      const int byte = (t * V + 8 * r) / 8;
      if (byte < (int)row_bytes) {
        s_mask[byte] = (uint8_t)mb;
        s_sign[byte] = (uint8_t)sb;
      }
    }
  }
  const float ktot = block_tree<WB>(lane_tree<RUNS>(rs), red);  // its barriers order the plane bytes
  const int nnz = block_sum<WB>(cnt, ired);
  const float alpha = nnz ? ktot / (float)nnz : 0.0f;
  if (blockIdx.x == 0) {
    if (o_mask)
      for (int i = t; i < (int)row_bytes; i += blockDim.x) {
        o_mask[i] = s_mask[i];
        o_sign[i] = s_sign[i];
      }
    if (o_alpha && t == 0) {
      o_alpha[0] = alpha;
      o_nnz[0] = nnz;
    }
  }

  // 3. the lane's activation words: p = mask ^ sign, s = sign
  uint32_t ap[NCH][4], as[NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int off = c * 1024 + lane * 16;
    u32x4 mm = u32x4{0, 0, 0, 0}, ss = u32x4{0, 0, 0, 0};
    if (cvalid[c]) {
      mm = *reinterpret_cast<const u32x4*>(s_mask + off);
      ss = *reinterpret_cast<const u32x4*>(s_sign + off);
    }
    ap[c][0] = mm.x ^ ss.x; ap[c][1] = mm.y ^ ss.y; ap[c][2] = mm.z ^ ss.z; ap[c][3] = mm.w ^ ss.w;
    as[c][0] = ss.x; as[c][1] = ss.y; as[c][2] = ss.z; as[c][3] = ss.w;
  }

  // 4. the weight stream (acc = nnz - 2 sum popc(bfi(w, mask ^ sign, sign)))
  for (int64_t n0 = wave * R; n0 < N; n0 += nwaves * R) {
    if (n0 != wave * R) load_w(n0);
    int c4[R];
#pragma unroll
    for (int r = 0; r < R; ++r) c4[r] = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t ww[4] = {w[r][c].x, w[r][c].y, w[r][c].z, w[r][c].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          c4[r] += __builtin_popcount((ww[q] & ap[c][q]) | (~ww[q] & as[c][q]));
      }
    wave_reduce_scatter_int<R>(c4);
    if (lane < R) {
      const int r = bitrev<2>(lane);
      const int64_t n = n0 + r;
      if (n < N) store_out<OUT>(Y, n, nnz - 2 * c4[0], alpha, OUT == (int)Elt::I32 ? 0.0f : w_alpha[n]);
    }
  }
}

template <int NCH, typename TX, int RUNS, int WB>
hipError_t launch_fused_row_nch(const GemmArgs& g, const TX* X, uint8_t* o_mask, uint8_t* o_sign,
                                float* o_alpha, int32_t* o_nnz, hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t waves_needed = (g.N + 3) / 4;
  int64_t blocks = (waves_needed + WB - 1) / WB;
  if (blocks > kFusedRowWaves / WB) blocks = kFusedRowWaves / WB;
  const dim3 grid((unsigned)blocks), block(WB * kWave);
  switch (g.y_dt) {
    case Elt::F32:
      hipLaunchKernelGGL((gemv_fused_row_kernel<NCH, TX, (int)Elt::F32, RUNS, WB>), grid, block, 0, stream,
                         X, (int)g.K, g.b_sign, g.b_alpha, g.N, row_bytes, g.Y, o_mask, o_sign,
                         o_alpha, o_nnz);
      break;
    case Elt::BF16:
      hipLaunchKernelGGL((gemv_fused_row_kernel<NCH, TX, (int)Elt::BF16, RUNS, WB>), grid, block, 0,
                         stream, X, (int)g.K, g.b_sign, g.b_alpha, g.N, row_bytes, g.Y, o_mask, o_sign,
                         o_alpha, o_nnz);
      break;
    default:
      hipLaunchKernelGGL((gemv_fused_row_kernel<NCH, TX, (int)Elt::I32, RUNS, WB>), grid, block, 0, stream,
                         X, (int)g.K, g.b_sign, g.b_alpha, g.N, row_bytes, g.Y, o_mask, o_sign,
                         o_alpha, o_nnz);
  }
  return hipGetLastError();
}

// Every block ternarizes the whole row, so the redundant ternarization work
// scales with the number of blocks: the launch takes the widest blocks (16, 8
// or 4 waves) that still give every compute unit a block, with at most
// kFusedRowWaves waves in the grid.  Threads hold RUNS runs of 8 values.
template <typename TX>
hipError_t launch_fused_row(const GemmArgs& g, const TX* X, uint8_t* o_mask, uint8_t* o_sign,
                            float* o_alpha, int32_t* o_nnz, hipStream_t stream) {
  int64_t P = 8;
  while (P < g.K) P <<= 1;
  const int64_t nch = ((g.K + 63) / 64 * 8 + 1023) / 1024;
  const int64_t waves_needed = (g.N + 3) / 4;
  // 16-wave blocks only for one-chunk rows: their 64-VGPR budget holds no more
  int wb = 4;
  if (nch <= 1 && waves_needed >= 16 * kFusedCUs) wb = 16;
  else if (waves_needed >= 8 * kFusedCUs) wb = 8;
#define BWTA_FR(NCH_, RUNS_, WB_) \
  return launch_fused_row_nch<NCH_, TX, RUNS_, WB_>(g, X, o_mask, o_sign, o_alpha, o_nnz, stream)
  if (nch <= 1) {  // P <= 8192
    if (wb == 16) BWTA_FR(1, 1, 16);
    if (wb == 8) BWTA_FR(1, 2, 8);
    BWTA_FR(1, 4, 4);
  }
  if (nch <= 2) {  // P <= 16384
    if (wb == 8) BWTA_FR(2, 4, 8);
    BWTA_FR(2, 8, 4);
  }
  if (wb == 8) BWTA_FR(4, 8, 8);
  BWTA_FR(4, 16, 4);
#undef BWTA_FR
}

template <int OUT>
hipError_t launch_gemm_pc_out(const GemmArgs& g, hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t tm = (g.M + PBM - 1) / PBM, tn = (g.N + PBN - 1) / PBN;
  const dim3 grid((unsigned)(tm * tn), 1, (unsigned)g.batch), block(256);
  if (g.b_mask)
    hipLaunchKernelGGL((gemm_popcount_kernel<true, OUT>), grid, block, 0, stream, g.a_mask, g.a_sign,
                       g.a_alpha, g.a_nnz, g.a_batch_rows, g.b_mask, g.b_sign, g.b_alpha,
                       g.b_batch_rows, g.M, g.N, row_bytes, (int)tn, g.Y, g.ldy, g.y_batch_stride);
  else
    hipLaunchKernelGGL((gemm_popcount_kernel<false, OUT>), grid, block, 0, stream, g.a_mask,
                       g.a_sign, g.a_alpha, g.a_nnz, g.a_batch_rows, g.b_mask, g.b_sign, g.b_alpha,
                       g.b_batch_rows, g.M, g.N, row_bytes, (int)tn, g.Y, g.ldy, g.y_batch_stride);
  return hipGetLastError();
}

template <int MB, int NCH, int OUT, bool RES = false>
hipError_t launch_gemv_cfg(const GemmArgs& g, int m_base, int m_count, hipStream_t stream) {
  // Four weight rows per wave (4 KiB of loads per 1 KiB chunk column): for
  // M = 1 this streams faster than 1, 2, 8 or 16 rows per wave.
  constexpr int R = 4;
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t waves_needed = (g.N + (RES ? 2 : R) - 1) / (RES ? 2 : R);
  int64_t blocks = (waves_needed + 3) / 4;
  const int64_t cap = 256 * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((gemv_popcount_kernel<MB, NCH, R, OUT, RES>), dim3((unsigned)blocks), dim3(256), 0,
                     stream, g.a_mask, g.a_sign, g.a_alpha, g.a_nnz, m_base, m_count, g.b_sign,
                     g.b_alpha, g.N, row_bytes, g.Y, g.ldy);
  return hipGetLastError();
}

template <int NCH, int OUT, bool RES = false>
hipError_t launch_gemv_nch(const GemmArgs& g, hipStream_t stream) {
  // activation registers: 8 * MB * NCH <= 128
  constexpr int MBMAX = 16 / NCH >= 4 ? 4 : (16 / NCH >= 2 ? 2 : 1);
  for (int64_t m0 = 0; m0 < g.M; m0 += MBMAX) {
    const int cnt = (int)(g.M - m0 < MBMAX ? g.M - m0 : MBMAX);
    hipError_t e;
    if (cnt == 1)
      e = launch_gemv_cfg<1, NCH, OUT, RES>(g, (int)m0, 1, stream);
    else if (cnt == 2 || MBMAX == 2)
      e = launch_gemv_cfg<(MBMAX >= 2 ? 2 : 1), NCH, OUT, RES>(g, (int)m0, cnt, stream);
    else
      e = launch_gemv_cfg<MBMAX, NCH, OUT, RES>(g, (int)m0, cnt, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int OUT, bool RES = false>
hipError_t launch_gemv_out(const GemmArgs& g, hipStream_t stream) {
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int64_t nch = (row_bytes + 1023) / 1024;
  if (nch <= 1) return launch_gemv_nch<1, OUT, RES>(g, stream);
  if (nch <= 2) return launch_gemv_nch<2, OUT, RES>(g, stream);
  if (nch <= 4) return launch_gemv_nch<4, OUT, RES>(g, stream);
  if (nch <= 8) return launch_gemv_nch<8, OUT, RES>(g, stream);
  return hipErrorInvalidValue;
}

// Two-plane products whose plane rows are one 64-bit word (K <= 64), the rows
// the FP4 kernel's 16-byte window does not take.  One thread per output column n
// holds the words of its two plane rows (64 (n / 32) + n % 32 and 32 further,
// consecutive for consecutive n) and walks a range of activation rows:
//   acc_i = popc(m) - 2 popc(m & (s ^ w_i)),
//   y = fl32(fl32(acc1 * fl32(aa * a1)) + fl32(acc2 * fl32(aa * a2))).
template <int OUT>
__global__ void __launch_bounds__(256)
residual_word_kernel(const uint64_t* __restrict__ a_mask, const uint64_t* __restrict__ a_sign,
                     const float* __restrict__ a_alpha, int64_t M,
                     const uint64_t* __restrict__ w_sign, const float* __restrict__ w_alpha,
                     int64_t N, void* __restrict__ Y, int64_t ldy, int64_t rows_per_block) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int64_t pn = 64 * (n >> 5) + (n & 31);
  const uint64_t w1 = w_sign[pn], w2 = w_sign[pn + 32];
  const float a1 = w_alpha[pn], a2 = w_alpha[pn + 32];
  const int64_t m0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t m1 = m0 + rows_per_block < M ? m0 + rows_per_block : M;
  for (int64_t m = m0; m < m1; ++m) {
    const uint64_t mk = a_mask[m], sg = a_sign[m];
    // (HIP's __popcll returns an unsigned int: count in int so nz - 2 c can go negative)
    const int nz = (int)__popcll(mk);
    const float acc1 = (float)(nz - 2 * (int)__popcll(mk & (sg ^ w1)));
    const float acc2 = (float)(nz - 2 * (int)__popcll(mk & (sg ^ w2)));
    const float aa = a_alpha[m];
    const float y = acc1 * (aa * a1) + acc2 * (aa * a2);
    if constexpr (OUT == (int)Elt::F32)
      static_cast<float*>(Y)[m * ldy + n] = y;
    else
      static_cast<__bf16*>(Y)[m * ldy + n] = (__bf16)y;
  }
}

template <int OUT>
hipError_t launch_residual_word_out(const GemmArgs& g, hipStream_t stream) {
  const int64_t N = g.N / 2;  // outputs
  int64_t rows = g.M < 16 ? g.M : 16;  // activation rows per block
  if ((g.M + rows - 1) / rows > 65535) rows = (g.M + 65534) / 65535;
  const int64_t gy = (g.M + rows - 1) / rows;
  hipLaunchKernelGGL(residual_word_kernel<OUT>, dim3((unsigned)((N + 255) / 256), (unsigned)gy),
                     dim3(256), 0, stream, reinterpret_cast<const uint64_t*>(g.a_mask),
                     reinterpret_cast<const uint64_t*>(g.a_sign), g.a_alpha, g.M,
                     reinterpret_cast<const uint64_t*>(g.b_sign), g.b_alpha, N, g.Y, g.ldy, rows);
  return hipGetLastError();
}

}  // namespace

// Two-plane product for K <= 64: g.N counts plane rows (twice the outputs, a
// multiple of 64), one 8-byte word per plane row.
hipError_t launch_gemm_residual_word(const GemmArgs& g, hipStream_t stream) {
  if (g.K > 64 || g.N % 64 != 0) return hipErrorInvalidValue;
  switch (g.y_dt) {
    case Elt::F32: return launch_residual_word_out<(int)Elt::F32>(g, stream);
    case Elt::BF16: return launch_residual_word_out<(int)Elt::BF16>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_popcount(const GemmArgs& g, hipStream_t stream) {
  switch (g.y_dt) {
    case Elt::F32: return launch_gemm_pc_out<(int)Elt::F32>(g, stream);
    case Elt::BF16: return launch_gemm_pc_out<(int)Elt::BF16>(g, stream);
    case Elt::I32: return launch_gemm_pc_out<(int)Elt::I32>(g, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_popcount(const GemmArgs& g, hipStream_t stream) {
  switch (g.y_dt) {
    case Elt::F32: return launch_gemv_out<(int)Elt::F32>(g, stream);
    case Elt::BF16: return launch_gemv_out<(int)Elt::BF16>(g, stream);
    case Elt::I32: return launch_gemv_out<(int)Elt::I32>(g, stream);
  }
  return hipErrorInvalidValue;
}

// Two-plane residual weights, M <= 16: g.N counts outputs (a multiple of 32),
// g.b_sign / g.b_alpha hold 2 g.N interleaved plane rows.
hipError_t launch_gemv_popcount_residual(const GemmArgs& g, hipStream_t stream) {
  if (g.N % 32 != 0) return hipErrorInvalidValue;
  switch (g.y_dt) {
    case Elt::F32: return launch_gemv_out<(int)Elt::F32, true>(g, stream);
    case Elt::BF16: return launch_gemv_out<(int)Elt::BF16, true>(g, stream);
    default: return hipErrorInvalidValue;
  }
}

// bwta_gemv_fused for one activation row (see gemv_fused_row_kernel):
// hipErrorNotSupported when the row does not fit its fast path (M != 1, K not a
// multiple of 8 or above kFusedMaxK, X not 16-byte aligned, ternary B).
hipError_t launch_gemv_fused_row(const GemmArgs& g, const void* X, Elt x_dt, uint8_t* o_mask,
                                 uint8_t* o_sign, float* o_alpha, int32_t* o_nnz,
                                 hipStream_t stream) {
  // Lanes read whole 16-byte words of a plane row (as gemv_popcount_kernel does,
  // under the same condition): row_bytes % 16 keeps them inside the weight rows.
  if (g.M != 1 || g.batch != 1 || g.b_mask || g.K % 8 != 0 || g.K > kFusedMaxK ||
      (g.K + 63) / 64 * 8 % 16 != 0 ||
      (x_dt != Elt::BF16 && g.K > kFusedMaxK / 2) || reinterpret_cast<uintptr_t>(X) % 16 != 0)
    return hipErrorNotSupported;
  return x_dt == Elt::BF16
             ? launch_fused_row(g, static_cast<const uint16_t*>(X), o_mask, o_sign, o_alpha, o_nnz,
                                stream)
             : launch_fused_row(g, static_cast<const float*>(X), o_mask, o_sign, o_alpha, o_nnz,
                                stream);
}

}  // namespace bwta
