// gemv_mfma.hip - decode GEMV / skinny GEMM (1 <= M <= 16) of binary weights
// W [N x K] and ternary activations A [M x K] on the FP4 matrix cores.
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract: bit-packed binary/ternary MatMul;
// decode is a pass over the 1-bit weights, so the kernel is judged by how close
// it streams them to HBM speed.
//
// Design:
// * v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 (e2m1) operands.  The weights are
//   the MFMA's A operand (16 weight rows per tile) and the M <= 16 activation
//   rows its B operand, so nothing is wasted for M = 16 and the VALU cost of
//   building operands does not grow with M.
// * Bit slices.  Lane (r, g) (r = lane % 16, g = lane / 16) holds, for chunk c
//   (64 bytes of every row), the words x = 0..3 at byte 64c + 16g + 4x of its
//   row.  MFMA e (0..3) of a chunk takes in nibble j of operand register x the
//   bit 4j + e of word x, for A and B alike, so A and B pair the same k.
//     weights: the sign bit b itself, w & (0x1.. << e) for e < 3 and
//              (w >> 1) & 0x4.. for e = 3, i.e. the values b * {0.5, 1, 2, 2},
//              brought to b by the A scale 2^{1, 0, -1, -1};
//     activations: t in {-1, 0, +1} as e2m1 (0x2 = 1, 0xA = -1), from
//              q01 = bfi(0x33.., m, s << 2), q23 = bfi(0x33.., m >> 2, s):
//              e = 0: (q01 << 1) & 0xA..,  1: q01 & 0xA..,
//              e = 2: (q23 << 1) & 0xA..,  3: q23 & 0xA..
//   So the MFMAs sum U = sum_k t_k b_k exactly (integers below 2^24), and with
//   s_k = 1 - 2 b_k the product is sum_k t_k s_k = T - 2U, T = sum_k t_k =
//   popc(mask) - 2 popc(sign) over the row, counted while staging.
// * Every wave owns one tile of 16 weight rows and one of S contiguous K ranges,
//   and walks its range in order (per load instruction: 16 rows x 64 contiguous
//   bytes).  It keeps kPF * kNB chunks of weight loads in flight from its first
//   instruction on: the whole range when it is short, a ring refilled as chunks
//   are consumed otherwise.  Ring slots past the range load from an offset the
//   buffer range check rejects, which returns zeros without touching memory, and
//   are not computed.
// * A block is R row groups x S waves (R * S <= 8), about one block per compute
//   unit.  It stages the activations of the whole K range in LDS once:
//     expanded (when 4 KiB per chunk fits): the B operands themselves, all 16
//       rows (zeros for rows m >= M and bytes past a row's end), lane-major per
//       (chunk, e), so each wave reads them with no VALU work;
//     raw otherwise: the M live rows' mask and sign words, lane-major per
//       (chunk, g); lanes of rows m >= M read a zeroed slot.  Each wave builds
//       its B operands.
//   The staging loads are issued before the weight loads (memory counters retire
//   in order) and the weight loads before the staging data is awaited.
// * Epilogue scales are requested first of all, so their latency hides under the
//   weight stream.  S = 1: each lane applies y = (T - 2U) * (alpha_a[m] *
//   alpha_w[n]) to its own 4 consecutive columns; S > 1: the partial tiles meet
//   in LDS first.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMaxW = 8;                // waves per block
constexpr int kPF = 4;                  // chunks per batch
constexpr int kNB = 2;                  // batches in flight
constexpr int kMaxSU = 8;               // staged 16-byte units per thread and plane
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every range check
constexpr size_t kMaxLds = 150 * 1024;

// s_waitcnt immediate for "vmcnt = 0" (expcnt and lgkmcnt at their no-wait
// maxima; vmcnt is split over bits 3:0 and 15:14).
constexpr int vmcnt_wait0() { return 0x0F70; }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which waits for every load in flight - here the whole weight stream.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A scale (E8M0) of slice e: b * {0.5, 1, 2, 2} times 2^{1, 0, -1, -1} is b.
__device__ __forceinline__ constexpr int weight_scale(int e) { return e == 0 ? 128 : e == 1 ? 127 : 126; }

__device__ __forceinline__ v4f mfma16(v4i a, v4i b, v4f c, int scale_a) {
  const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
  const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, scale_a, 0, 127);
}

// Weight slice e of 4 words.
template <int E>
__device__ __forceinline__ v4i weight_slice(v4u w) {
  v4i o;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    o[x] = (int)(E == 3 ? (w[x] >> 1) & 0x44444444u : w[x] & (0x11111111u << E));
  return o;
}

// Activation slices e = 0..3 of one (mask, sign) word pair.  The merges go
// through bitop3 (0xE4: S2 ? S0 : S1) so that the compiler keeps this form.
__device__ __forceinline__ void act_slices(uint32_t m, uint32_t s, uint32_t (&o)[4]) {
  const uint32_t q01 = __builtin_amdgcn_bitop3_b32(m, s << 2, 0x33333333u, 0xE4);
  const uint32_t q23 = __builtin_amdgcn_bitop3_b32(m >> 2, s, 0x33333333u, 0xE4);
  o[0] = (q01 << 1) & 0xAAAAAAAAu;
  o[1] = q01 & 0xAAAAAAAAu;
  o[2] = (q23 << 1) & 0xAAAAAAAAu;
  o[3] = q23 & 0xAAAAAAAAu;
}

// LDS layout.  Expanded: chunk c, slice e, slot s at ((c * 4 + e) * 64 + s) * 16,
// plus one cleared chunk.
// Raw: plane p (0 mask, 1 sign) at p * plane, slot (c, g, m) at
// ((c * 4 + g) * M + m) * 16 within it, then 32 zeroed bytes.  After either:
// per wave the 16 row sums T (int), then the S > 1 exchange.
struct LdsLayout {
  uint32_t plane, zero_off, t_off, x_off, total;
};

__host__ __device__ inline LdsLayout lds_layout(bool expanded, int chunks, int M, int S, int R,
                                                int accs = 1) {
  LdsLayout l;
  l.plane = (uint32_t)chunks * 4u * (uint32_t)M * 16u;
  l.zero_off = 2 * l.plane;
  l.t_off = expanded ? (uint32_t)(chunks + 1) * 4096u : l.zero_off + 32u;
  l.x_off = l.t_off + kMaxW * 16u * 4u;
  l.total = l.x_off + (S > 1 ? (uint32_t)(S * R * accs) * 64u * 16u : 0u);
  return l;
}

// ---------------------------------------------------------------------------
// Fused ternarization (XT != 0): the block ternarizes its M activation rows
// itself, from fp32 (XT = 1) or bf16 (XT = 2) values, by the rule of
// bwta_ternarize_pack, and writes the packed bits straight into the raw staging
// layout of its chunk range; so one launch does the decode linear's whole work.
//
// Reduction order.  With P the power of two at or above K, NT threads (a power
// of two, NT <= blockDim) each own the aligned run [t V, t V + V) of V = P / NT
// values (V >= 8, zeros past K).  A thread folds its run 8 values at a time into
// a binary-counter stack (a perfect tree over the run), the 64 lanes of a wave
// meet in a butterfly (lane bit 0 first) and the waves in a pairwise LDS tree, so
// every total is the perfect pairwise tree over the zero-padded row, bit for bit.
template <typename TX>
struct XRun {
  static constexpr int kWords = sizeof(TX) == 2 ? 4 : 8;  // 32-bit words per 8 values
  static constexpr int kGroup = 16 / kWords;              // runs loaded per batch
};

__device__ __forceinline__ uint32_t x_bits(const uint32_t* w, int j, float) { return w[j]; }
__device__ __forceinline__ uint32_t x_bits(const uint32_t* w, int j, uint16_t) {
  return (w[j >> 1] >> (16 * (j & 1))) << 16;
}

template <typename TX>
__device__ __forceinline__ void x_load_run(const TX* __restrict__ row, int64_t k0, int K, bool vec,
                                           uint32_t (&w)[XRun<TX>::kWords]) {
  constexpr int NW = XRun<TX>::kWords;
  if (vec && k0 + 8 <= K) {
#pragma unroll
    for (int v = 0; v < NW / 4; ++v) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(row + k0 + v * (16 / (int)sizeof(TX)));
#pragma unroll
      for (int x = 0; x < 4; ++x) w[4 * v + x] = u[x];
    }
  } else {
#pragma unroll
    for (int x = 0; x < NW; ++x) w[x] = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (k0 + j < K) {
        uint32_t b;
        if constexpr (sizeof(TX) == 4)
          b = __float_as_uint(row[k0 + j]);
        else
          b = (uint32_t)row[k0 + j];
        if constexpr (sizeof(TX) == 4)
          w[j] = b;
        else
          w[j >> 1] |= b << (16 * (j & 1));
      }
    }
  }
}

// Binary-counter merge of run n's tree node into the stack (levels 0..kXStack-1).
// A thread folds at most 128 runs (V <= 1024 values: P <= 65536 over NT >= 64
// threads, or P < 512), so 9 levels suffice.
constexpr int kXStack = 9;
__device__ __forceinline__ void stack_push(float (&st)[kXStack], int n, float node) {
  bool open = true;
#pragma unroll
  for (int l = 0; l < kXStack; ++l) {
    const bool merge = open && ((n >> l) & 1);
    if (merge) node = st[l] + node;
    if (open && !merge) {
      st[l] = node;
      open = false;
    }
  }
}
__device__ __forceinline__ float stack_root(const float (&st)[kXStack], int runs) {
  float root = 0.0f;
#pragma unroll
  for (int l = 0; l < kXStack; ++l)
    if ((runs >> l) & 1) root = st[l] + root;
  return root;
}

// Sum over the NT participating threads: butterfly inside each wave, then the
// pairwise tree over the waves' sums through `red` (NT / 64 entries, at most 8).
__device__ __forceinline__ float block_tree(float v, int NT, float* red) {
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int lanes = NT < kWave ? NT : kWave;
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((1 << b) < lanes) v = v + __shfl_xor(v, 1 << b, kWave);
  const int nw = NT < kWave ? 1 : NT / kWave;
  if (lane == 0 && wid < nw) red[wid] = v;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return tree16(red, nw);
}
__device__ __forceinline__ int block_isum(int v, int NT, int* red) {
  const int lane = __lane_id();
  const int wid = threadIdx.x / kWave;
  const int lanes = NT < kWave ? NT : kWave;
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((1 << b) < lanes) v += __shfl_xor(v, 1 << b, kWave);
  const int nw = NT < kWave ? 1 : NT / kWave;
  if (lane == 0 && wid < nw) red[wid] = v;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  int s = 0;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// Fallback for rows whose run of values per thread does not fit the register
// budget of fused_ternarize: one row at a time, the values read twice.
template <typename TX>
__device__ __forceinline__ void fused_ternarize_rows(const TX* __restrict__ X, int64_t ldx, int M, int K, int row_bytes,
                                int kc0, int chunks, uint8_t* smem, uint32_t plane_bytes,
                                int* tw, float* s_alpha, int* s_nnz, float* red, int* ired,
                                uint8_t* o_mask, uint8_t* o_sign, float* o_alpha, int32_t* o_nnz,
                                bool out_planes, bool out_scales) {
  constexpr int NW = XRun<TX>::kWords, NG = XRun<TX>::kGroup;
  int P = 1;
  while (P < K) P <<= 1;
  int Bp = 1;
  while (2 * Bp <= (int)blockDim.x) Bp <<= 1;
  const int NT = Bp < (P >= 8 ? P / 8 : 1) ? Bp : (P >= 8 ? P / 8 : 1);
  const int V = P / NT;       // values per thread (>= 8 unless P < 8)
  const int runs = (V + 7) / 8;
  const int t = threadIdx.x;
  const bool part = t < NT;
  const int64_t kt = (int64_t)t * V;  // first value of the thread's run
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((ldx * (int64_t)sizeof(TX)) % 16 == 0) &&
                   (K % 8 == 0);
  const int lo = kc0 * 512, hi = (kc0 + chunks) * 512;  // the block's k range
  for (int m = 0; m < M; ++m) {
    const TX* row = X + (int64_t)m * ldx;
    // pass 1: tree(|x|)
    float st[kXStack];
#pragma unroll
    for (int l = 0; l < kXStack; ++l) st[l] = 0.0f;
    for (int g0 = 0; g0 < runs; g0 += NG) {
      uint32_t w[NG][NW];
#pragma unroll
      for (int i = 0; i < NG; ++i)
        if (part && g0 + i < runs && kt + 8 * (g0 + i) < K)
          x_load_run<TX>(row, kt + 8 * (g0 + i), K, vec, w[i]);
        else
#pragma unroll
          for (int x = 0; x < NW; ++x) w[i][x] = 0u;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (g0 + i < runs) {
          float a[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) a[j] = __uint_as_float(x_bits(w[i], j, TX{}) & 0x7FFFFFFFu);
          stack_push(st, g0 + i, lane_tree<8>(a));
        }
      }
    }
    const float total = block_tree(part ? stack_root(st, runs) : 0.0f, NT, red);
    const float mu = total / (float)K;
    const uint32_t uthr = __float_as_uint(0.5f * mu);
    // pass 2: threshold, bits, tree(kept |x|), counts
#pragma unroll
    for (int l = 0; l < kXStack; ++l) st[l] = 0.0f;
    int cnt = 0, tpart = 0;
    for (int g0 = 0; g0 < runs; g0 += NG) {
      uint32_t w[NG][NW];
#pragma unroll
      for (int i = 0; i < NG; ++i)
        if (part && g0 + i < runs && kt + 8 * (g0 + i) < K)
          x_load_run<TX>(row, kt + 8 * (g0 + i), K, vec, w[i]);
        else
#pragma unroll
          for (int x = 0; x < NW; ++x) w[i][x] = 0u;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (g0 + i < runs) {
          float kept[8];
          uint32_t mb = 0, sb = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t ux = x_bits(w[i], j, TX{});
            const uint32_t ua = ux & 0x7FFFFFFFu;
            const uint32_t keep = (uthr - ua) >> 31;  // |x| > thr (non-negative bit patterns)
            kept[j] = __uint_as_float(ua & (0u - keep));
            mb |= keep << j;
            sb |= (keep & (ux >> 31)) << j;
          }
          stack_push(st, g0 + i, lane_tree<8>(kept));
          const int64_t k0 = kt + 8 * (g0 + i);
          cnt += __builtin_popcount(mb);
          if (part && k0 >= lo && k0 < hi && k0 < (int64_t)row_bytes * 8) {
            const int kl = (int)k0 - lo;  // local bit offset
            const int cl = kl >> 9, gg = (kl >> 7) & 3, byte = (kl & 127) >> 3;
            const uint32_t off = (uint32_t)(((cl * 4 + gg) * M + m) * 16 + byte);
            smem[off] = (uint8_t)mb;
            smem[plane_bytes + off] = (uint8_t)sb;
            tpart += __builtin_popcount(mb) - 2 * __builtin_popcount(sb);
            if (out_planes) {
              o_mask[(int64_t)m * row_bytes + (k0 >> 3)] = (uint8_t)mb;
              o_sign[(int64_t)m * row_bytes + (k0 >> 3)] = (uint8_t)sb;
            }
          }
        }
      }
    }
    if (tpart) atomicAdd(&tw[m], tpart);
    // Rows shorter than 32 values: the runs cover bytes [0, (P + 7) / 8) of the
    // 8-byte row; the rest of the plane row is zero padding.
    if (out_planes && t == 0)
      for (int b = (P + 7) / 8; b < row_bytes && b < hi / 8; ++b) {
        o_mask[(int64_t)m * row_bytes + b] = 0;
        o_sign[(int64_t)m * row_bytes + b] = 0;
      }
    const float ktot = block_tree(part ? stack_root(st, runs) : 0.0f, NT, red + 8);
    const int ctot = block_isum(part ? cnt : 0, NT, ired);
    const float alpha = ctot ? ktot / (float)ctot : 0.0f;
    if (t == 0) {
      s_alpha[m] = alpha;
      s_nnz[m] = ctot;
      if (out_scales) {
        o_alpha[m] = alpha;
        o_nnz[m] = ctot;
      }
    }
  }
}

// The prologue.  Rows m < M of X (row m at X + m * ldx) become the raw staging
// planes of local chunks [0, chunks) = global chunks [kc0, kc0 + chunks) (the
// caller cleared them), the row sums T of that range go to the wave counters
// tw (atomic adds), and alpha_a / nnz of the whole row to s_alpha / s_nnz.  With
// out_planes the block also writes the planes of its range (and, with
// out_scales, alpha and nnz) to global memory.
//
// Rows go in groups of G whose runs all fit 8 register slots per thread (slot i
// holds run i % runs of row i / runs): one round of loads per group, the run
// trees of each row added pairwise in registers (runs is a power of two, so
// the row's slots form one aligned sub-tree), one butterfly per row, and two
// block barriers per group.  red, red2, ired hold 16 rows x 8 waves each.
template <typename TX>
__device__ __forceinline__ void fused_ternarize(const TX* __restrict__ X, int64_t ldx, int M, int K,
                                                int row_bytes, int kc0, int chunks, uint8_t* smem,
                                                uint32_t plane_bytes, int* tw, float* s_alpha,
                                                int* s_nnz, float* red, float* red2, int* ired,
                                                uint8_t* o_mask, uint8_t* o_sign, float* o_alpha,
                                                int32_t* o_nnz, bool out_planes, bool out_scales) {
  constexpr int NW = XRun<TX>::kWords;
  constexpr int SLOTS = 8;  // runs held at once (32 registers of bf16, 64 of fp32)
  int P = 1;
  while (P < K) P <<= 1;
  int Bp = 1;
  while (2 * Bp <= (int)blockDim.x) Bp <<= 1;
  const int NT = Bp < (P >= 8 ? P / 8 : 1) ? Bp : (P >= 8 ? P / 8 : 1);
  const int V = P / NT;
  const int runs = (V + 7) / 8;  // a power of two
  const int t = threadIdx.x;
  if (t < 16) s_alpha[t] = 0.0f;  // rows m >= M read 0 (ordered by the barriers below)
  // Vector loads only (16-byte aligned rows, K a multiple of 8), and the runs of
  // a row within the slots; other inputs take the per-row fallback.
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) &&
                   ((ldx * (int64_t)sizeof(TX)) % 16 == 0) && (K % 8 == 0);
  if (runs > SLOTS || !vec) {
    fused_ternarize_rows<TX>(X, ldx, M, K, row_bytes, kc0, chunks, smem, plane_bytes, tw, s_alpha,
                             s_nnz, red, ired, o_mask, o_sign, o_alpha, o_nnz, out_planes,
                             out_scales);
    return;
  }
  const int lane = __lane_id();
  const int wid = t / kWave;
  const bool part = t < NT;
  const int nw = NT < kWave ? 1 : NT / kWave;
  const int lanes = NT < kWave ? NT : kWave;
  const int64_t kt = (int64_t)t * V;
  const int lo = kc0 * 512, hi = (kc0 + chunks) * 512;
  const int G = SLOTS / runs;
  const int lr = 31 - __builtin_clz(runs);  // runs = 2^lr: slot i is run i & (runs - 1) of row i >> lr
  auto barrier = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  auto butterfly = [&](float v) {
#pragma unroll
    for (int b = 0; b < 6; ++b)
      if ((1 << b) < lanes) v = v + __shfl_xor(v, 1 << b, kWave);
    return v;
  };
  for (int m0 = 0; m0 < M; m0 += G) {
    const int gm = M - m0 < G ? M - m0 : G;  // rows in this group
    uint32_t w[SLOTS][NW];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int gi = i >> lr, r = i & (runs - 1);
      const int64_t k0 = kt + 8 * r;
      if (part && gi < gm && k0 < K) {
        const TX* src = X + (int64_t)(m0 + gi) * ldx + k0;
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) {
          const u32x4 u = *reinterpret_cast<const u32x4*>(src + v * (16 / (int)sizeof(TX)));
#pragma unroll
          for (int x = 0; x < 4; ++x) w[i][4 * v + x] = u[x];
        }
      } else {
#pragma unroll
        for (int x = 0; x < NW; ++x) w[i][x] = 0u;
      }
    }
    // pass 1: |x| run trees, then pairwise over each row's runs
    float n[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = __uint_as_float(x_bits(w[i], j, TX{}) & 0x7FFFFFFFu);
      n[i] = lane_tree<8>(a);
    }
#pragma unroll
    for (int h = 1; h < SLOTS; h <<= 1)
      if (2 * h <= runs)
#pragma unroll
        for (int i = 0; i + h < SLOTS; i += 2 * h) n[i] = n[i] + n[i + h];
#pragma unroll
    for (int i = 0; i < SLOTS; i += 1) {
      if ((i & (runs - 1)) == 0 && (i >> lr) < gm) {
        const float v = butterfly(part ? n[i] : 0.0f);
        if (lane == 0 && wid < nw) red[(i >> lr) * 8 + wid] = v;
      }
    }
    barrier();
    // the rows' thresholds, each computed once
    uint32_t thr_g[SLOTS];
#pragma unroll
    for (int g = 0; g < SLOTS; ++g)
      thr_g[g] = g < gm ? __float_as_uint(0.5f * (tree16(red + g * 8, nw) / (float)K)) : 0u;
    // pass 2 (values still in registers): threshold, bits, kept trees, counts
    float kn[SLOTS];
    int cnt[SLOTS], tpart[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int gi = i >> lr, r = i & (runs - 1);
      const int m = m0 + gi;
      kn[i] = 0.0f;
      cnt[i] = 0;
      tpart[i] = 0;
      if (gi < gm) {
        uint32_t uthr = thr_g[0];
#pragma unroll
        for (int g = 1; g <= i; ++g) uthr = gi == g ? thr_g[g] : uthr;
        float kept[8];
        uint32_t mb = 0, sb = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t ux = x_bits(w[i], j, TX{});
          const uint32_t ua = ux & 0x7FFFFFFFu;
          const uint32_t keep = (uthr - ua) >> 31;  // |x| > thr (non-negative bit patterns)
          kept[j] = __uint_as_float(ua & (0u - keep));
          mb |= keep << j;
          sb |= (keep & (ux >> 31)) << j;
        }
        kn[i] = lane_tree<8>(kept);
        cnt[i] = __builtin_popcount(mb);
        const int64_t k0 = kt + 8 * r;
        if (part && k0 >= lo && k0 < hi && k0 < (int64_t)row_bytes * 8) {
          const int kl = (int)k0 - lo;
          const int cl = kl >> 9, gg = (kl >> 7) & 3, byte = (kl & 127) >> 3;
          const uint32_t off = (uint32_t)(((cl * 4 + gg) * M + m) * 16 + byte);
          smem[off] = (uint8_t)mb;
          smem[plane_bytes + off] = (uint8_t)sb;
          tpart[i] = __builtin_popcount(mb) - 2 * __builtin_popcount(sb);
        }
      }
    }
#pragma unroll
    for (int h = 1; h < SLOTS; h <<= 1)
      if (2 * h <= runs)
#pragma unroll
        for (int i = 0; i + h < SLOTS; i += 2 * h) {
          kn[i] = kn[i] + kn[i + h];
          cnt[i] = cnt[i] + cnt[i + h];
          tpart[i] = tpart[i] + tpart[i + h];
        }
#pragma unroll
    for (int i = 0; i < SLOTS; i += 1) {
      if ((i & (runs - 1)) == 0 && (i >> lr) < gm) {
        const float v = butterfly(part ? kn[i] : 0.0f);
        int c = part ? cnt[i] : 0, tp = part ? tpart[i] : 0;
#pragma unroll
        for (int b = 0; b < 6; ++b)
          if ((1 << b) < lanes) {
            c += __shfl_xor(c, 1 << b, kWave);
            tp += __shfl_xor(tp, 1 << b, kWave);
          }
        if (lane == 0 && wid < nw) {
          red2[(i >> lr) * 8 + wid] = v;
          ired[(i >> lr) * 8 + wid] = c;
          if (tp) atomicAdd(&tw[m0 + (i >> lr)], tp);  // one add per wave and row
        }
      }
    }
    barrier();
    if (out_planes) {
      // The group's rows of the staged planes (its chunk range, zero padding
      // included) to global memory, 16 or 8 bytes at a time.
      const int units = chunks * 4 * gm;
      for (int u = t; u < units; u += blockDim.x) {
        const int gi = u % gm, q = u / gm, cl = q >> 2, gg = q & 3;
        const int64_t byte = (int64_t)(kc0 + cl) * 64 + gg * 16;
        if (byte >= row_bytes) continue;
        const uint32_t off = (uint32_t)(((cl * 4 + gg) * M + m0 + gi) * 16);
        const int64_t dst = (int64_t)(m0 + gi) * row_bytes + byte;
        const uint64_t* ms = reinterpret_cast<const uint64_t*>(smem + off);
        const uint64_t* ss = reinterpret_cast<const uint64_t*>(smem + plane_bytes + off);
        *reinterpret_cast<uint64_t*>(o_mask + dst) = ms[0];
        *reinterpret_cast<uint64_t*>(o_sign + dst) = ss[0];
        if (byte + 8 < row_bytes) {
          *reinterpret_cast<uint64_t*>(o_mask + dst + 8) = ms[1];
          *reinterpret_cast<uint64_t*>(o_sign + dst + 8) = ss[1];
        }
      }
    }
    if (t < gm) {
      const float ktot = tree16(red2 + t * 8, nw);
      int ctot = 0;
      for (int q = 0; q < nw; ++q) ctot += ired[t * 8 + q];
      const float alpha = ctot ? ktot / (float)ctot : 0.0f;
      s_alpha[m0 + t] = alpha;
      s_nnz[m0 + t] = ctot;
      if (out_scales) {
        o_alpha[m0 + t] = alpha;
        o_nnz[m0 + t] = ctot;
      }
    }
  }
}

// RES: two-plane residual weights (planes interleaved in groups of 32 rows), N
// counts outputs.  The wave of output tile o (16 outputs) streams both of its
// plane tiles - rows 64 (o / 2) + 16 (o % 2) and 32 rows further - with half as
// many chunks per batch (the same bytes in flight), multiplies both by the same
// activation operands, and the epilogue writes
// y = (T - 2 U1) (alpha_a alpha1) + (T - 2 U2) (alpha_a alpha2).
//
// XB: K split across blocks (a workspace is given).  blockIdx.y = ky picks the
// block's contiguous chunk range, one of gridDim.y; the block stages only that
// range, every wave (S = 1) multiplies its tile over it, stores the exact int32
// partial T_ky - 2 U_ky of its 16 x 16 outputs in its slot of the workspace and
// counts itself in the tile's arrival counter.  The last of the gridDim.y blocks
// to arrive adds the partials (integers: the order does not matter), applies the
// epilogue and returns the counter to zero, so no block ever waits for another.
//
// XT: the activations arrive as fp32 (1) or bf16 (2) rows in io.X and the block
// ternarizes them itself (fused_ternarize) into the raw staging layout; a_mask,
// a_sign and a_alpha are not read.
//
// XP: fp32 (1) or bf16 (2) rows in io.X, each ternarized once (produce_rows)
// into the exchange buffers io.x_*, which the blocks then stage as in the plain
// kernel (see "Ternarize-once decode"); a_mask, a_sign, a_alpha are not read.
struct FusedIO {
  const void* X;
  int64_t ldx;
  int K;             // logical row length
  uint8_t* o_mask;   // optional outputs (NULL: not written)
  uint8_t* o_sign;
  float* o_alpha;
  int32_t* o_nnz;
  int* flags;        // XP: row flags [0, 16) and the arrival counter [16]
  int spin;          // XP: polls of the flags before a block ternarizes the rows itself
  // XP: the exchange buffers (workspace).  Plain pointers on purpose: the
  // kernel's restrict-qualified a_* arguments promise memory no one writes.
  uint8_t* x_mask;
  uint8_t* x_sign;
  float* x_alpha;
  int32_t* x_nnz;
  int splits;        // XP: the cross-block K split's part count (the grid is 1-D)
};

// ---------------------------------------------------------------------------
// Ternarize-once decode (XP = 1 for fp32 rows, 2 for bf16; one launch, with a
// workspace).  The exchange buffers (io.x_mask, x_sign, x_alpha, x_nnz, in the
// workspace) receive each row's planes and scale from one block: the grid's
// first M blocks (dispatched first) do nothing else; block m ternarizes row m
// by the rule of bwta_ternarize_pack, stores it with device-coherent stores
// (they reach memory, past this XCD's L2, without a cache flush; the optional
// outputs o_* get plain copies) and raises the row's flag once they have
// completed.  Every other block issues the first revolution of its weight ring
// (the loads land while it waits), polls the flags with device-coherent loads
// until all M are up, and stages the planes exactly as the plain decode kernel
// does.  Those loads may go through L2: no block reads the exchange buffers
// before it has seen their flags, so no L2 holds an older copy of them within
// the launch, and launches start with the L2s invalidated.  The wait is bounded: a block
// that has polled `spin` times ternarizes every row itself (the same values, so
// the repeated stores change nothing) and goes on, so no block waits on another
// without end whatever the order blocks start in.  At its end each block counts
// itself in; the last one returns the flags and the counter to zero.
constexpr int kXPFlags = 16;  // index of the arrival counter among the flags

// The producer's block sums: the butterfly over the participating lanes by
// xor_lane (DPP and swizzle moves, no LDS round trip per level), the same pairs
// in the same order as block_tree, then the waves' tree through LDS.  The pair
// form reduces the kept-value tree and the count behind one barrier.
__device__ __forceinline__ float p_butterfly(float v, int lanes) {
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((1 << b) < lanes) v = v + xor_lane(v, 1 << b);
  return v;
}
__device__ __forceinline__ int p_butterfly(int v, int lanes) {
#pragma unroll
  for (int b = 0; b < 6; ++b)
    if ((1 << b) < lanes) v += xor_lane(v, 1 << b);
  return v;
}
__device__ __forceinline__ float p_block_tree(float v, int NT, float* red) {
  const int lane = __lane_id(), wid = threadIdx.x / kWave;
  v = p_butterfly(v, NT < kWave ? NT : kWave);
  const int nw = NT < kWave ? 1 : NT / kWave;
  if (lane == 0 && wid < nw) red[wid] = v;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return tree16(red, nw);
}
__device__ __forceinline__ void p_block_pair(float v, int c, int NT, float* red, int* ired,
                                             float& vt, int& ct) {
  const int lane = __lane_id(), wid = threadIdx.x / kWave;
  const int lanes = NT < kWave ? NT : kWave;
  v = p_butterfly(v, lanes);
  c = p_butterfly(c, lanes);
  const int nw = NT < kWave ? 1 : NT / kWave;
  if (lane == 0 && wid < nw) {
    red[wid] = v;
    ired[wid] = c;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  vt = tree16(red, nw);
  int s = 0;
  for (int w = 0; w < nw; ++w) s += ired[w];
  ct = s;
}

// REG: rows of at most 8 runs per thread keep their values in registers between
// the passes (one round of loads); otherwise, and always with REG = false (the
// path of a block that ternarizes the rows itself while its weight loads hold
// registers), the values are read twice.
template <typename TX, bool REG>
__device__ void produce_row(const TX* __restrict__ row, int K, int row_bytes, uint8_t* lds,
                            float* red, int* ired, uint8_t* g_mask, uint8_t* g_sign,
                            float* g_alpha, int32_t* g_nnz, uint8_t* u_mask, uint8_t* u_sign,
                            float* u_alpha, int32_t* u_nnz, bool vec) {
  constexpr int NW = XRun<TX>::kWords, NG = XRun<TX>::kGroup;
  constexpr int kRegRuns = 8;  // runs a thread holds in registers between the passes
  int P = 1;
  while (P < K) P <<= 1;
  int Bp = 1;
  while (2 * Bp <= (int)blockDim.x) Bp <<= 1;
  const int NT = Bp < (P >= 8 ? P / 8 : 1) ? Bp : (P >= 8 ? P / 8 : 1);
  const int V = P / NT;
  const int runs = (V + 7) / 8;
  const int t = threadIdx.x;
  const bool part = t < NT;
  const int64_t kt = (int64_t)t * V;
  auto load = [&](int n, uint32_t (&w)[NW]) {  // run n of the thread (zeros past the row)
    if (part && n < runs && kt + 8 * n < K)
      x_load_run<TX>(row, kt + 8 * n, K, vec, w);
    else
#pragma unroll
      for (int x = 0; x < NW; ++x) w[x] = 0u;
  };
  auto abs_node = [&](const uint32_t (&w)[NW]) {  // pass 1: tree(|x|) of one run
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __uint_as_float(x_bits(w, j, TX{}) & 0x7FFFFFFFu);
    return lane_tree<8>(a);
  };
  uint32_t uthr = 0;
  int cnt = 0;
  auto kept_node = [&](int n, const uint32_t (&w)[NW]) {  // pass 2 of one run
    float kept[8];
    uint32_t mb = 0, sb = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t ux = x_bits(w, j, TX{});
      const uint32_t ua = ux & 0x7FFFFFFFu;
      const uint32_t keep = (uthr - ua) >> 31;  // |x| > thr (non-negative bit patterns)
      kept[j] = __uint_as_float(ua & (0u - keep));
      mb |= keep << j;
      sb |= (keep & (ux >> 31)) << j;
    }
    cnt += __builtin_popcount(mb);
    const int64_t k0 = kt + 8 * n;
    if (part && k0 < (int64_t)row_bytes * 8) {
      lds[k0 >> 3] = (uint8_t)mb;
      lds[row_bytes + (k0 >> 3)] = (uint8_t)sb;
    }
    return lane_tree<8>(kept);
  };
  // the row's planes in LDS (mask, then sign), cleared: bytes no run covers stay 0
  uint32_t* lw = reinterpret_cast<uint32_t*>(lds);
  for (int i = t; i < row_bytes / 2; i += blockDim.x) lw[i] = 0u;
  float st[kXStack];
#pragma unroll
  for (int l = 0; l < kXStack; ++l) st[l] = 0.0f;
  float ktot;
  if (REG && runs <= kRegRuns) {
    // one round of loads; the values stay in registers for pass 2
    uint32_t w[kRegRuns][NW];
#pragma unroll
    for (int n = 0; n < kRegRuns; ++n) load(n, w[n]);
#pragma unroll
    for (int n = 0; n < kRegRuns; ++n)
      if (n < runs) stack_push(st, n, abs_node(w[n]));
    // (its barrier also orders the clearing before the plane bytes below)
    const float total = p_block_tree(part ? stack_root(st, runs) : 0.0f, NT, red);
    uthr = __float_as_uint(0.5f * (total / (float)K));
#pragma unroll
    for (int l = 0; l < kXStack; ++l) st[l] = 0.0f;
#pragma unroll
    for (int n = 0; n < kRegRuns; ++n)
      if (n < runs) stack_push(st, n, kept_node(n, w[n]));
  } else {
    // long runs: the values read twice, NG runs at a time
    for (int g0 = 0; g0 < runs; g0 += NG) {
      uint32_t w[NG][NW];
#pragma unroll
      for (int i = 0; i < NG; ++i) load(g0 + i, w[i]);
#pragma unroll
      for (int i = 0; i < NG; ++i)
        if (g0 + i < runs) stack_push(st, g0 + i, abs_node(w[i]));
    }
    const float total = p_block_tree(part ? stack_root(st, runs) : 0.0f, NT, red);
    uthr = __float_as_uint(0.5f * (total / (float)K));
#pragma unroll
    for (int l = 0; l < kXStack; ++l) st[l] = 0.0f;
    for (int g0 = 0; g0 < runs; g0 += NG) {
      uint32_t w[NG][NW];
#pragma unroll
      for (int i = 0; i < NG; ++i) load(g0 + i, w[i]);
#pragma unroll
      for (int i = 0; i < NG; ++i)
        if (g0 + i < runs) stack_push(st, g0 + i, kept_node(g0 + i, w[i]));
    }
  }
  // (its barrier orders the plane bytes before the word reads below)
  int ctot;
  p_block_pair(part ? stack_root(st, runs) : 0.0f, part ? cnt : 0, NT, red + 8, ired, ktot, ctot);
  const float alpha = ctot ? ktot / (float)ctot : 0.0f;
  const int words = row_bytes / 4;
  for (int i = t; i < words; i += blockDim.x) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(g_mask) + i, lw[i], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(reinterpret_cast<uint32_t*>(g_sign) + i, lw[words + i], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (u_mask)
    for (int i = t; i < words; i += blockDim.x) {
      reinterpret_cast<uint32_t*>(u_mask)[i] = lw[i];
      reinterpret_cast<uint32_t*>(u_sign)[i] = lw[words + i];
    }
  if (t == 0) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(g_alpha), __float_as_uint(alpha),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(g_nnz, ctot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (u_alpha) {
      *u_alpha = alpha;
      *u_nnz = ctot;
    }
  }
  // every store of the block has completed before the barrier, and the LDS
  // planes are read before anything overwrites them
  __builtin_amdgcn_s_waitcnt(vmcnt_wait0());
  lds_barrier();
}

// Rows m = first, first + step, ... < M of X into the exchange buffers, each
// followed by its flag (after the row's stores have completed).  The flag
// stores complete before the block's arrival count (xp_arrive).
template <typename TX, bool REG>
__device__ void produce_rows(const FusedIO& io, int M, int row_bytes, int first, int step,
                             uint8_t* lds, float* red, int* ired, uint8_t* x_mask,
                             uint8_t* x_sign, float* x_alpha, int32_t* x_nnz) {
  const TX* X = static_cast<const TX*>(io.X);
  const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) &&
                   ((io.ldx * (int64_t)sizeof(TX)) % 16 == 0) && (io.K % 8 == 0);
  for (int m = first; m < M; m += step) {
    const int64_t ro = (int64_t)m * row_bytes;
    produce_row<TX, REG>(X + (int64_t)m * io.ldx, io.K, row_bytes, lds, red, ired, x_mask + ro,
                         x_sign + ro, x_alpha + m, x_nnz + m, io.o_mask ? io.o_mask + ro : nullptr,
                         io.o_mask ? io.o_sign + ro : nullptr, io.o_alpha ? io.o_alpha + m : nullptr,
                         io.o_alpha ? io.o_nnz + m : nullptr, vec);
    if (threadIdx.x == 0)  // (completed before the block counts itself in)
      __hip_atomic_store(io.flags + m, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int S, bool X, int OUT, bool RES = false, bool XB = false, int XT = 0, int XP = 0>
__global__ void __launch_bounds__(kMaxW * kWave)
gemv_mfma_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                 const float* __restrict__ a_alpha, int M, const uint8_t* __restrict__ w_sign,
                 const float* __restrict__ w_alpha, int64_t N, int row_bytes,
                 void* __restrict__ Y, int64_t ldy, int* __restrict__ ws_ctr,
                 int* __restrict__ ws_part, FusedIO io) {
  static_assert(!XB || (S == 1 && !RES), "the cross-block split runs unsplit one-plane waves");
  static_assert(XT == 0 || (!X && !RES), "fused ternarization stages raw one-plane operands");
  static_assert(XP == 0 || (XT == 0 && !RES), "ternarize-once decode stages one-plane operands");
  __shared__ float s_alpha[16], s_red[16 * 8], s_red2[16 * 8];
  __shared__ int s_nnz[16], s_ired[16 * 8], s_xp;
  typedef typename std::conditional<XP == 1, float, uint16_t>::type XPT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int W = blockDim.x / kWave;
  const int R = W / S;  // row groups per block
  const int lane = __lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rg = wid / S, ks = wid - rg * S;
  const int r = lane & 15;
  const int g = lane >> 4;
  static_assert(!RES || OUT != (int)Elt::I32, "two-plane products are scaled");
  constexpr int PF = RES ? kPF / 2 : kPF;  // chunks per batch and plane
  constexpr int RING = PF * kNB;
  // XP: a 1-D grid whose first M blocks only ternarize; block M + c is the
  // consumer (c % cblocks, c / cblocks) of the plain 2-D grid.
  const int nblk = (int)(gridDim.x * gridDim.y);
  const int nsplit = XB ? (XP != 0 ? io.splits : (int)gridDim.y) : 1;
  const int cblocks = XP != 0 ? (nblk - M) / nsplit : (int)gridDim.x;
  const int c_lin = XP != 0 ? (int)blockIdx.x - M : 0;
  const int bx = XP != 0 ? c_lin % cblocks : (int)blockIdx.x;
  const int by = XP != 0 ? c_lin / cblocks : (int)blockIdx.y;
  // The block is past its wait (and its flag stores have completed): count it
  // in; the last one clears the flags.
  auto xp_arrive = [&]() {
    if (threadIdx.x == 0) {
      __builtin_amdgcn_s_waitcnt(vmcnt_wait0());
      const int old = __hip_atomic_fetch_add(io.flags + kXPFlags, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      if (old == nblk - 1) {
        for (int m = 0; m < M; ++m)
          __hip_atomic_store(io.flags + m, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(io.flags + kXPFlags, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  if constexpr (XP != 0) {
    if ((int)blockIdx.x < M) {  // 0. a producing block: its row, then nothing else
      produce_rows<XPT, true>(io, M, row_bytes, (int)blockIdx.x, M, smem, s_red, s_ired, io.x_mask,
                              io.x_sign, io.x_alpha, io.x_nnz);
      xp_arrive();
      return;
    }
  }
  const int64_t ot = (int64_t)bx * R + rg;  // output tile
  const int64_t n0 = ot * 16;
  const int64_t p1 = RES ? 64 * (ot >> 1) + 16 * (ot & 1) : n0;  // its (first) plane rows
  const int64_t rows_left = N - n0;
  const int rows_here = rows_left <= 0 ? 0 : (rows_left < 16 ? (int)rows_left : 16);
  // The block's chunk range [kc0, kc0 + chunks) (all of the row unless XB); LDS
  // holds it at local chunk indices 0 .. chunks - 1.
  const int all_chunks = (row_bytes + 63) / 64;
  const int ky = XB ? by : 0;
  const int kc0 = XB ? all_chunks * ky / nsplit : 0;
  const int chunks = XB ? all_chunks * (ky + 1) / nsplit - kc0 : all_chunks;
  const int c0 = kc0 + chunks * ks / S;
  const int c1 = kc0 + chunks * (ks + 1) / S;
  const LdsLayout L = lds_layout(X, chunks, M, S, R, RES ? 2 : 1);
  int* tsum = reinterpret_cast<int*>(smem + L.t_off);
  // the planes the block stages: the exchange buffers (XP) or the arguments
  const uint8_t* const st_mask = XP != 0 ? io.x_mask : a_mask;
  const uint8_t* const st_sign = XP != 0 ? io.x_sign : a_sign;

  // 1. Epilogue scales.  Items: S = 1, the lanes of the own wave; S > 1, item
  //    p = threadIdx.x (row group p / 64, lane p % 64) when p < R * 64.
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  const int p_item = S == 1 ? lane : (int)threadIdx.x;
  const bool item_ok = S == 1 || p_item < R * kWave;
  const int64_t nb_item = S == 1 ? n0 : ((int64_t)bx * R + p_item / kWave) * 16;
  const int l_item = p_item % kWave;
  v4f ab = v4f{0.0f, 0.0f, 0.0f, 0.0f}, ab2 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float aa = 0.0f;
  if constexpr (OUT != (int)Elt::I32) {
    const __amdgpu_buffer_rsrc_t ars = checked_rsrc(w_alpha, (uint32_t)((RES ? 2 : 1) * N * 4));
    const int64_t n = nb_item + 4 * (l_item >> 4);
    // plane row of output n (RES: interleaved groups of 32)
    const int64_t pn = RES ? 64 * (n >> 5) + (n & 31) : n;
    // n is a multiple of 4; the 4-byte range check zeroes the floats past N.
    ab = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                     ars, (int)(n < N ? (uint32_t)(pn * 4) : kOOB), 0, 0));
    if constexpr (RES)
      ab2 = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                        ars, (int)(n < N ? (uint32_t)((pn + 32) * 4) : kOOB), 0, 0));
    if constexpr (XT == 0 && XP == 0) {
      const __amdgpu_buffer_rsrc_t aars = checked_rsrc(a_alpha, (uint32_t)M * 4u);
      aa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         aars, (int)((l_item & 15) * 4), 0, 0));
    }
  }
  // 2. Staging loads, 16 bytes per plane and unit u = (m * chunks + c) * 4 + g
  //    over the M live rows (row-major, so one load instruction reads whole
  //    64-byte pieces of a row).
  const int units = chunks * 4 * M;
  // float quotients are exact after a +-1 fix-up for u < 2^24
  auto fdiv = [](int u, int d, float inv) {
    int q = (int)((float)u * inv);
    q += (q + 1) * d <= u ? 1 : 0;
    q -= q * d > u ? 1 : 0;
    return q;
  };
  const float inv_c = 1.0f / (float)chunks;
  auto unit_pos = [&](int u, int& m, int& c, int& gg) {
    gg = u & 3;
    const int q = u >> 2;
    m = fdiv(q, chunks, inv_c);
    c = q - m * chunks;
  };
  const int nsu = XT ? 0 : (units + (int)blockDim.x - 1) / (int)blockDim.x;  // rounds, uniform
  const __amdgpu_buffer_rsrc_t mrs = checked_rsrc(st_mask, (uint32_t)M * (uint32_t)row_bytes);
  const __amdgpu_buffer_rsrc_t srs = checked_rsrc(st_sign, (uint32_t)M * (uint32_t)row_bytes);
  v4u sm[kMaxSU], ss[kMaxSU];
  auto stage_loads = [&]() {
#pragma unroll
    for (int k = 0; k < kMaxSU; ++k) {
      if (k < nsu) {
        const int u = (int)threadIdx.x + k * (int)blockDim.x;
        int m, c, gg;
        unit_pos(u, m, c, gg);
        const uint32_t off = u < units ? (uint32_t)(m * row_bytes + 64 * (kc0 + c) + 16 * gg) : kOOB;
        sm[k] = __builtin_amdgcn_raw_buffer_load_b128(mrs, (int)off, 0, 0);
        ss[k] = __builtin_amdgcn_raw_buffer_load_b128(srs, (int)off, 0, 0);
      }
    }
  };
  if constexpr (XP == 0) stage_loads();

  // 3. Weight ring: slot (b, i) holds chunk base + b * kPF + i of the current
  //    revolution.  Batch 0 goes out now, the others once the activations are
  //    staged: a wave that queues many loads stalls on issue until the memory
  //    pipeline drains, and it has to get to the staging first.
  const __amdgpu_buffer_rsrc_t wrs =
      checked_rsrc(w_sign + (rows_here ? p1 * row_bytes : 0), (uint32_t)(rows_here * row_bytes));
  const __amdgpu_buffer_rsrc_t wrs2 = checked_rsrc(
      w_sign + (RES && rows_here ? (p1 + 32) * row_bytes : 0), (uint32_t)(rows_here * row_bytes));
  const uint32_t w_lane = (uint32_t)(r * row_bytes + 16 * g);
  v4u wr[kNB][PF], wr2[kNB][PF];
  auto issue = [&](int b, int cb) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int c = cb + i;
      const int off = (int)(c < c1 ? w_lane + 64u * (uint32_t)c : kOOB);
      wr[b][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
      if constexpr (RES) wr2[b][i] = __builtin_amdgcn_raw_buffer_load_b128(wrs2, off, 0, 0);
    }
  };
  issue(0, c0);
  if constexpr (XP != 0) {
#pragma unroll
    for (int b = 1; b < kNB; ++b) issue(b, c0 + b * PF);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XP != 0) {
    // Wait (bounded) for every row's flag under the first revolution of the
    // weight ring.
    if (wid == 0) {
      int ok = 0;
      for (int it = 0;; ++it) {
        const int v =
            lane < M ? __hip_atomic_load(io.flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
        ok = __all(v != 0);
        if (ok || it >= io.spin) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane == 0) s_xp = ok;
    }
    lds_barrier();
    if (!s_xp)  // not all rows ready in time: ternarize them here as well
      produce_rows<XPT, false>(io, M, row_bytes, 0, 1, smem, s_red, s_ired, io.x_mask, io.x_sign,
                               io.x_alpha, io.x_nnz);
    // no load of the exchange buffers may move above the wait
    __asm__ volatile("" ::: "memory");
    if constexpr (OUT != (int)Elt::I32) {
      const int m = l_item & 15;
      aa = m < M ? io.x_alpha[m] : 0.0f;
    }
    stage_loads();
  }

  // 4. Staging stores (they wait for the staging loads only) and row sums T,
  //    accumulated per wave in its own 16 LDS counters (cleared by the wave
  //    itself, so no barrier is needed before the adds).  Units past the first
  //    kMaxSU rounds (long rows over few waves) are loaded and stored one at a
  //    time.  Expanded operands go to slot g * 16 + (m ^ h(c, g)) of their
  //    (chunk, e) group, h = 4 (c & 1) + g: the 8 lanes of one store (4 g, 2
  //    chunks) and of one read (8 rows) hit distinct bank groups.  Lanes of rows
  //    m >= M read a cleared extra chunk.
  int* tw = tsum + wid * 16;
  if (lane < 16) tw[lane] = 0;
  if constexpr (XT != 0) {
    // Clear the raw planes (bytes no run covers must read 0), then ternarize.
    for (uint32_t z = threadIdx.x * 16u; z < L.zero_off + 32u; z += blockDim.x * 16u)
      *reinterpret_cast<v4u*>(smem + z) = v4u{0u, 0u, 0u, 0u};
    const bool first = blockIdx.x == 0;
    if constexpr (XT == 1)
      fused_ternarize<float>(static_cast<const float*>(io.X), io.ldx, M, io.K,
                             row_bytes, kc0, chunks, smem, L.plane, tw, s_alpha, s_nnz, s_red,
                             s_red2, s_ired, io.o_mask, io.o_sign, io.o_alpha, io.o_nnz,
                             first && io.o_mask, first && ky == 0 && io.o_alpha);
    else
      fused_ternarize<uint16_t>(static_cast<const uint16_t*>(io.X), io.ldx, M, io.K,
                                row_bytes, kc0, chunks, smem, L.plane, tw, s_alpha, s_nnz, s_red,
                                s_red2, s_ired, io.o_mask, io.o_sign, io.o_alpha, io.o_nnz,
                                first && io.o_mask, first && ky == 0 && io.o_alpha);
  }
  auto stage_unit = [&](int u, v4u vm, v4u vs) {
    int m, c, gg;
    unit_pos(u, m, c, gg);
    const int valid = row_bytes - 64 * (kc0 + c) - 16 * gg;  // bytes of this unit inside the row
    if (valid < 16) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vm[x] = 4 * x < valid ? vm[x] : 0u;
        vs[x] = 4 * x < valid ? vs[x] : 0u;
      }
    }
    int t = 0;
#pragma unroll
    for (int x = 0; x < 4; ++x) t += __builtin_popcount(vm[x]) - 2 * __builtin_popcount(vs[x]);
    atomicAdd(&tw[m], t);
    if constexpr (X) {
      uint32_t o[4][4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        uint32_t sl[4];
        act_slices(vm[x], vs[x], sl);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e][x] = sl[e];
      }
      const int slot = gg * 16 + (m ^ (((c & 1) << 2) | gg));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<v4u*>(smem + ((c * 4 + e) * 64 + slot) * 16) =
            v4u{o[e][0], o[e][1], o[e][2], o[e][3]};
    } else {
      const uint32_t slot = (uint32_t)((c * 4 + gg) * M + m) * 16u;
      *reinterpret_cast<v4u*>(smem + slot) = vm;
      *reinterpret_cast<v4u*>(smem + L.plane + slot) = vs;
    }
  };
#pragma unroll
  for (int k = 0; k < kMaxSU; ++k) {
    const int u = (int)threadIdx.x + k * (int)blockDim.x;
    if (k < nsu && u < units) stage_unit(u, sm[k], ss[k]);
  }
  for (int u = (int)threadIdx.x + kMaxSU * (int)blockDim.x; XT == 0 && u < units;
       u += (int)blockDim.x) {
    int m, c, gg;
    unit_pos(u, m, c, gg);
    const uint32_t off = (uint32_t)(m * row_bytes + 64 * (kc0 + c) + 16 * gg);
    stage_unit(u, __builtin_amdgcn_raw_buffer_load_b128(mrs, (int)off, 0, 0),
               __builtin_amdgcn_raw_buffer_load_b128(srs, (int)off, 0, 0));
  }
  if constexpr (X) {
    for (int z = threadIdx.x; z < 256; z += blockDim.x)  // the extra chunk
      *reinterpret_cast<v4u*>(smem + (uint32_t)chunks * 4096u + z * 16) = v4u{0u, 0u, 0u, 0u};
  } else if constexpr (XT == 0) {
    if (threadIdx.x < 2)
      *reinterpret_cast<v4u*>(smem + L.zero_off + 16 * threadIdx.x) = v4u{0u, 0u, 0u, 0u};
  }
  if constexpr (XP == 0) {
#pragma unroll
    for (int b = 1; b < kNB; ++b) issue(b, c0 + b * PF);
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  if constexpr (XT != 0) aa = s_alpha[l_item & 15];  // 0 for rows m >= M (never stored)

  // 5. Main loop.  Raw B operand of lane (r, g) for chunk c: slot (c, g, r) when
  //    r < M, else the zeroed slot (mask 0 makes every product 0).
  const bool live = r < M;
  const uint32_t am_base = X ? 0u : live ? (uint32_t)(g * M + r) * 16u : L.zero_off;
  const uint32_t as_base = live ? L.plane + am_base : L.zero_off;
  const uint32_t a_step = X ? 0u : live ? (uint32_t)(4 * M) * 16u : 0u;
  v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f}, acc2 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int b, int cb) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int c = cb + i;
      if (c < c1) {  // uniform
        const int cl = c - kc0;  // staged (local) chunk
        const uint32_t ao = am_base + (uint32_t)cl * a_step;
        v4i bop[4];
        if constexpr (X) {
          // lane slot of chunk c (rows m >= M: the cleared extra chunk)
          const uint32_t xo = live ? (uint32_t)cl * 4096u +
                                         (uint32_t)(g * 16 + (r ^ (((cl & 1) << 2) | g))) * 16u
                                   : (uint32_t)chunks * 4096u;
#pragma unroll
          for (int e = 0; e < 4; ++e) bop[e] = *reinterpret_cast<const v4i*>(smem + xo + e * 1024);
        } else {
          const v4u am = *reinterpret_cast<const v4u*>(smem + ao);
          const v4u as = *reinterpret_cast<const v4u*>(smem + as_base + (uint32_t)cl * a_step);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            uint32_t sl[4];
            act_slices(am[x], as[x], sl);
#pragma unroll
            for (int e = 0; e < 4; ++e) bop[e][x] = (int)sl[e];
          }
        }
        const v4u w = wr[b][i];
        acc = mfma16(weight_slice<0>(w), bop[0], acc, weight_scale(0));
        acc = mfma16(weight_slice<1>(w), bop[1], acc, weight_scale(1));
        acc = mfma16(weight_slice<2>(w), bop[2], acc, weight_scale(2));
        acc = mfma16(weight_slice<3>(w), bop[3], acc, weight_scale(3));
        if constexpr (RES) {
          const v4u w2 = wr2[b][i];
          acc2 = mfma16(weight_slice<0>(w2), bop[0], acc2, weight_scale(0));
          acc2 = mfma16(weight_slice<1>(w2), bop[1], acc2, weight_scale(1));
          acc2 = mfma16(weight_slice<2>(w2), bop[2], acc2, weight_scale(2));
          acc2 = mfma16(weight_slice<3>(w2), bop[3], acc2, weight_scale(3));
        }
      }
    }
  };
  // Full revolutions refill their slots; the last one issues nothing, so the
  // epilogue does not wait behind loads of chunks past the range.
  int cb = c0;
  for (; cb + RING < c1; cb += RING) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      compute(b, cb + b * PF);
      issue(b, cb + b * PF + RING);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int b = 0; b < kNB; ++b) compute(b, cb + b * PF);

  // 6. Epilogue.  Element u of the U tile in lane l: activation row m = l % 16,
  //    column n_base + 4 (l / 16) + u; the product is T[m] - 2U.
  // emit: the products acc1 (and acc2, RES) of lane l's 4 outputs, exact
  // integers in fp32, through the epilogue to Y.
  auto emit = [&](int l, v4f acc1, v4f acc2v, int64_t nb) {
    const int m = l & 15;
    const int64_t n = nb + 4 * (l >> 4);
    if (m >= M || n >= N) return;
    uint32_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float accf = acc1[u];
      if constexpr (OUT == (int)Elt::I32) {
        o[u] = (uint32_t)(int)accf;
      } else {
        float y = accf * (aa * ab[u]);
        if constexpr (RES) {
          const float y2 = acc2v[u] * (aa * ab2[u]);
          y = y + y2;
        }
        o[u] = OUT == (int)Elt::F32 ? __float_as_uint(y)
                                    : (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y);
      }
    }
    char* yp = static_cast<char*>(Y) + ((int64_t)m * ldy + n) * ES;
    if (n + 4 <= N && (reinterpret_cast<uintptr_t>(yp) % (4 * ES)) == 0) {
      if constexpr (ES == 4)
        *reinterpret_cast<v4u*>(yp) = v4u{o[0], o[1], o[2], o[3]};
      else
        *reinterpret_cast<uint2*>(yp) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (n + u >= N) break;
        if constexpr (ES == 4)
          reinterpret_cast<uint32_t*>(yp)[u] = o[u];
        else
          reinterpret_cast<uint16_t*>(yp)[u] = (uint16_t)o[u];
      }
    }
  };
  // store: lane l's MFMA sums U (and U2) of the block's whole range, T - 2U.
  auto store = [&](int l, v4f u4, v4f u4b, int64_t nb) {
    const int m = l & 15;
    int tm = 0;
    for (int w2 = 0; w2 < W; ++w2) tm += tsum[w2 * 16 + m];
    const float t = (float)tm;
    v4f a1, a2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a1[u] = t - 2.0f * u4[u];  // exact: integers below 2^24
      a2[u] = t - 2.0f * u4b[u];
    }
    emit(l, a1, a2, nb);
  };

  if constexpr (XB) {
    if (rows_here > 0) {  // wave-uniform; tiles past N take no part in any split
      const int m = lane & 15;
      int tm = 0;
      for (int w2 = 0; w2 < W; ++w2) tm += tsum[w2 * 16 + m];
      v4i part;
#pragma unroll
      for (int u = 0; u < 4; ++u) part[u] = tm - 2 * (int)acc[u];  // exact integers
      // The partial goes to this split's slot of the tile with device-coherent
      // stores (agent-scope atomic stores: sc1, visible to every XCD once
      // complete, with no write-back or invalidation of the XCD's L2 as a fence
      // would do); after they have completed (the wait) the block counts itself
      // in, and the last block reads the other slots with device-coherent loads.
      const int64_t tiles_all = (N + 15) / 16;
      auto slot = [&](int k2) {
        return reinterpret_cast<uint64_t*>(ws_part + ((k2 * tiles_all + ot) * kWave + lane) * 4);
      };
      uint64_t* mine = slot(ky);
      __hip_atomic_store(mine, (uint64_t)(uint32_t)part[0] | ((uint64_t)(uint32_t)part[1] << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(mine + 1, (uint64_t)(uint32_t)part[2] | ((uint64_t)(uint32_t)part[3] << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(vmcnt_wait0());
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(ws_ctr + ot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __shfl(old, 0, kWave);
      if (old == nsplit - 1) {  // every other split's slot is complete
        v4i sum = part;
        for (int k2 = 0; k2 < nsplit; ++k2) {
          if (k2 == ky) continue;
          const uint64_t* o2 = slot(k2);
          const uint64_t lo = __hip_atomic_load(o2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t hi = __hip_atomic_load(o2 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sum += v4i{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi,
                     (int)(uint32_t)(hi >> 32)};
        }
        if (lane == 0)  // the counter is zero again for the next call
          __hip_atomic_store(ws_ctr + ot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v4f a1;
#pragma unroll
        for (int u = 0; u < 4; ++u) a1[u] = (float)sum[u];  // |acc| <= K < 2^24: exact
        emit(lane, a1, a1, n0);
      }
    }
  } else if constexpr (S == 1) {
    if (rows_here > 0) store(lane, acc, acc2, n0);
  } else {
    // Cross-wave sum of the S partial tiles of each row group (and plane).
    v4f* xbuf = reinterpret_cast<v4f*>(smem + L.x_off);
    v4f* xbuf2 = xbuf + S * R * kWave;
    xbuf[wid * kWave + lane] = acc;
    if constexpr (RES) xbuf2[wid * kWave + lane] = acc2;
    lds_barrier();
    if (item_ok) {
      const int grp = p_item / kWave;
      v4f sum = xbuf[(grp * S) * kWave + l_item];
      for (int k2 = 1; k2 < S; ++k2) sum += xbuf[(grp * S + k2) * kWave + l_item];
      v4f sum2 = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (RES) {
        sum2 = xbuf2[(grp * S) * kWave + l_item];
        for (int k2 = 1; k2 < S; ++k2) sum2 += xbuf2[(grp * S + k2) * kWave + l_item];
      }
      store(l_item, sum, sum2, nb_item);
    }
  }
  if constexpr (XP != 0) xp_arrive();
}

// Launch geometry for one group of mg activation rows.
struct Geometry {
  int S, R;
  bool X;
  int64_t blocks;
  size_t lds;
  bool fits;
};

Geometry geometry(int64_t N, int64_t row_bytes, int64_t mg, int accs = 1) {
  Geometry q;
  const int64_t chunks = (row_bytes + 63) / 64;
  const int64_t tiles = (N + 15) / 16;
  // Split K (contiguous ranges of at least 8 chunks) until there are 1536 or
  // more waves, then take about one block per compute unit.
  q.S = 1;
  while (q.S < kMaxW && tiles * q.S < 1536 && chunks >= 16 * q.S) q.S *= 2;
  int64_t R = (tiles + 255) / 256;
  if (R < 1) R = 1;
  if (R > kMaxW / q.S) R = kMaxW / q.S;
  q.R = (int)R;
  q.blocks = (tiles + R - 1) / R;
  q.X = (size_t)lds_layout(true, (int)chunks, (int)mg, q.S, q.R, accs).total <= kMaxLds;
  q.lds = lds_layout(q.X, (int)chunks, (int)mg, q.S, q.R, accs).total;
  q.fits = q.lds <= kMaxLds;
  return q;
}

// The cross-block K split (XB).  Where the in-block plan splits K over S waves
// (fewer than 1536 tiles), P blocks take contiguous chunk ranges instead, each
// staging only its range (LLaMA2-70B down, K = 28672: 28 KiB of planes per block
// at M = 16 instead of 112 KiB, and expanded B operands instead of raw words).
// The workspace starts with a fixed region of kCtrBytes for the arrival
// counters (one per tile, zero between calls: the last block of a tile clears
// its counter), followed by P int32 partial tiles of 16 x 16 per output tile.
// The counter region is the same for every shape, so a later call, whatever its
// tile count, finds its counters zero (partials never reach into it).
struct Split {
  bool use = false;
  int P = 1, R = 1;
  bool X = false;
  int64_t blocks = 0;
  size_t lds = 0, ctr_bytes = 0, ws_bytes = 0;
};

constexpr int64_t kMaxSplitTiles = 4096;  // P x tiles: at most 4 MiB of partials
constexpr size_t kCtrBytes = 8192;        // the region that is zero between calls
constexpr size_t kFlagBytes = 256;        // its last bytes: the fused decode's row flags

Split split_plan(int64_t M, int64_t N, int64_t row_bytes) {
  Split sp;
  // From 8 activation rows on: there the staged planes are a large share of a
  // block's bytes (70B down at M = 16: 10.8 us split against 14.4 us); at M = 4
  // the partials' round trip costs more than it saves (10.5 against 9.1 us).
  if (M < 8 || M > 16 || N >= ((int64_t)1 << 29)) return sp;
  const Geometry q1 = geometry(N, row_bytes, M);
  const int64_t tiles = (N + 15) / 16;
  const int64_t chunks = (row_bytes + 63) / 64;
  int P = q1.S;
  while (P > 1 && tiles * P > kMaxSplitTiles) P /= 2;
  if (P < 2 || tiles * 4 > (int64_t)(kCtrBytes - kFlagBytes)) return sp;
  const int64_t cb = (chunks + P - 1) / P;  // the largest range
  int64_t R = (tiles * P + 255) / 256;
  if (R < 1) R = 1;
  if (R > kMaxW) R = kMaxW;
  sp.P = P;
  sp.R = (int)R;
  sp.blocks = (tiles + R - 1) / R;
  sp.X = (size_t)lds_layout(true, (int)cb, (int)M, 1, sp.R).total <= kMaxLds;
  sp.lds = lds_layout(sp.X, (int)cb, (int)M, 1, sp.R).total;
  if (sp.lds > kMaxLds) return Split{};
  sp.ctr_bytes = kCtrBytes;
  sp.ws_bytes = sp.ctr_bytes + (size_t)P * (size_t)tiles * 1024;
  sp.use = true;
  return sp;
}

// io: the fused ternarization's rows (XT != 0; offset here to the group's rows).
template <int S, bool X, int OUT, bool RES = false, bool XB = false, int XT = 0, int XP = 0>
hipError_t launch_s(const GemmArgs& g, const Geometry& q, int64_t m0, int64_t mg,
                    int64_t row_bytes, hipStream_t stream, int splits = 1, int* ctr = nullptr,
                    int* part = nullptr, FusedIO io = FusedIO{}) {
  auto kfn = gemv_mfma_kernel<S, X, OUT, RES, XB, XT, XP>;
  hipError_t e = hipFuncSetAttribute((const void*)kfn,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)q.lds);
  if (e != hipSuccess) return e;
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  if constexpr (XT != 0) {
    io.X = static_cast<const char*>(io.X) + m0 * io.ldx * (XT == 1 ? 4 : 2);
    if (io.o_mask) io.o_mask += m0 * row_bytes;
    if (io.o_sign) io.o_sign += m0 * row_bytes;
    if (io.o_alpha) io.o_alpha += m0;
    if (io.o_nnz) io.o_nnz += m0;
  }
  const uint8_t* am = g.a_mask ? g.a_mask + m0 * row_bytes : nullptr;
  const uint8_t* as = g.a_sign ? g.a_sign + m0 * row_bytes : nullptr;
  if constexpr (XP != 0) io.splits = splits;
  const dim3 grid = XP != 0 ? dim3((unsigned)(mg + q.blocks * splits))
                            : dim3((unsigned)q.blocks, (unsigned)splits);
  hipLaunchKernelGGL(kfn, grid,
                     dim3((unsigned)(q.S * q.R * kWave)), q.lds, stream, am, as,
                     g.a_alpha ? g.a_alpha + m0 : nullptr, (int)mg, g.b_sign, g.b_alpha, g.N,
                     (int)row_bytes, static_cast<char*>(g.Y) + m0 * g.ldy * ES, g.ldy, ctr, part,
                     io);
  return hipGetLastError();
}

// Fused decode (XT = 1 fp32, 2 bf16 activations): raw staging only; the same
// cross-block split as launch_out when a workspace is given, else groups of
// activation rows whose raw planes fit in LDS.
template <int OUT, int XT>
hipError_t launch_fused(const GemmArgs& g, const FusedIO& io, hipStream_t stream) {
  if (g.N >= (int64_t)1 << 29) return hipErrorInvalidValue;  // 32-bit offsets
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const Split sp = g.ws ? split_plan(g.M, g.N, row_bytes) : Split{};
  if (sp.use) {
    if (g.ws_bytes < sp.ws_bytes) return hipErrorInvalidValue;  // checked by the caller
    const int64_t chunks = (row_bytes + 63) / 64;
    const int64_t cb = (chunks + sp.P - 1) / sp.P;
    Geometry q;
    q.S = 1;
    q.R = sp.R;
    q.X = false;
    q.blocks = sp.blocks;
    q.lds = lds_layout(false, (int)cb, (int)g.M, 1, sp.R).total;
    if (q.lds > kMaxLds) return hipErrorInvalidValue;
    int* ctr = static_cast<int*>(g.ws);
    int* part = reinterpret_cast<int*>(static_cast<char*>(g.ws) + sp.ctr_bytes);
    return launch_s<1, false, OUT, false, true, XT>(g, q, 0, g.M, row_bytes, stream, sp.P, ctr,
                                                    part, io);
  }
  auto raw = [&](int64_t mg) {
    Geometry q = geometry(g.N, row_bytes, mg);
    q.X = false;
    q.lds = lds_layout(false, (int)((row_bytes + 63) / 64), (int)mg, q.S, q.R).total;
    q.fits = q.lds <= kMaxLds;
    return q;
  };
  int64_t mg = g.M;
  while (mg > 1 && !raw(mg).fits) mg = (mg + 1) / 2;
  for (int64_t m0 = 0; m0 < g.M; m0 += mg) {
    const int64_t cnt = g.M - m0 < mg ? g.M - m0 : mg;
    const Geometry q = raw(cnt);
    if (!q.fits) return hipErrorInvalidValue;
    hipError_t e;
    switch (q.S) {
      case 1: e = launch_s<1, false, OUT, false, false, XT>(g, q, m0, cnt, row_bytes, stream, 1, nullptr, nullptr, io); break;
      case 2: e = launch_s<2, false, OUT, false, false, XT>(g, q, m0, cnt, row_bytes, stream, 1, nullptr, nullptr, io); break;
      case 4: e = launch_s<4, false, OUT, false, false, XT>(g, q, m0, cnt, row_bytes, stream, 1, nullptr, nullptr, io); break;
      default: e = launch_s<8, false, OUT, false, false, XT>(g, q, m0, cnt, row_bytes, stream, 1, nullptr, nullptr, io); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Ternarize-once decode (XP = 1 fp32, 2 bf16 rows): one launch over all M rows
// on the plain decode plan (the cross-block split where g.ws has one), with LDS
// for a producing block's row planes at least.  hipErrorNotSupported when the
// rows' staging does not fit one launch.  io.x_* are the exchange buffers.
template <int OUT, int XP>
hipError_t launch_xp(const GemmArgs& g, const FusedIO& io, hipStream_t stream) {
  if (g.N >= (int64_t)1 << 29) return hipErrorInvalidValue;  // 32-bit offsets
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const size_t prod = (size_t)(2 * row_bytes);
  const Split sp = g.ws ? split_plan(g.M, g.N, row_bytes) : Split{};
  if (sp.use) {
    if (g.ws_bytes < sp.ws_bytes) return hipErrorInvalidValue;
    Geometry q;
    q.S = 1;
    q.R = sp.R;
    q.X = sp.X;
    q.blocks = sp.blocks;
    q.lds = std::max(sp.lds, prod);
    q.fits = q.lds <= kMaxLds;
    if (!q.fits) return hipErrorNotSupported;
    int* ctr = static_cast<int*>(g.ws);
    int* part = reinterpret_cast<int*>(static_cast<char*>(g.ws) + sp.ctr_bytes);
    return sp.X ? launch_s<1, true, OUT, false, true, 0, XP>(g, q, 0, g.M, row_bytes, stream,
                                                             sp.P, ctr, part, io)
                : launch_s<1, false, OUT, false, true, 0, XP>(g, q, 0, g.M, row_bytes, stream,
                                                              sp.P, ctr, part, io);
  }
  Geometry q = geometry(g.N, row_bytes, g.M);
  if (!q.fits) return hipErrorNotSupported;
  q.lds = std::max(q.lds, prod);
  if (q.lds > kMaxLds) return hipErrorNotSupported;
#define BWTA_XP_S(SS)                                                                          \
  return q.X ? launch_s<SS, true, OUT, false, false, 0, XP>(g, q, 0, g.M, row_bytes, stream, 1,  \
                                                           nullptr, nullptr, io)               \
             : launch_s<SS, false, OUT, false, false, 0, XP>(g, q, 0, g.M, row_bytes, stream, 1, \
                                                            nullptr, nullptr, io)
  switch (q.S) {
    case 1: BWTA_XP_S(1);
    case 2: BWTA_XP_S(2);
    case 4: BWTA_XP_S(4);
    default: BWTA_XP_S(8);
  }
#undef BWTA_XP_S
}

template <bool X, int OUT, bool RES = false>
hipError_t launch_x(const GemmArgs& g, const Geometry& q, int64_t m0, int64_t mg,
                    int64_t row_bytes, hipStream_t stream) {
  switch (q.S) {
    case 1: return launch_s<1, X, OUT, RES>(g, q, m0, mg, row_bytes, stream);
    case 2: return launch_s<2, X, OUT, RES>(g, q, m0, mg, row_bytes, stream);
    case 4: return launch_s<4, X, OUT, RES>(g, q, m0, mg, row_bytes, stream);
    default: return launch_s<8, X, OUT, RES>(g, q, m0, mg, row_bytes, stream);
  }
}

template <int OUT, bool RES = false>
hipError_t launch_out(const GemmArgs& g, hipStream_t stream) {
  if ((RES ? 2 : 1) * g.N >= (int64_t)1 << 29) return hipErrorInvalidValue;  // 32-bit offsets
  const int64_t row_bytes = (g.K + 63) / 64 * 8;
  const int accs = RES ? 2 : 1;
  if constexpr (!RES) {
    const Split sp = g.ws ? split_plan(g.M, g.N, row_bytes) : Split{};
    if (sp.use) {
      if (g.ws_bytes < sp.ws_bytes) return hipErrorInvalidValue;  // checked by the caller
      Geometry q;
      q.S = 1;
      q.R = sp.R;
      q.X = sp.X;
      q.blocks = sp.blocks;
      q.lds = sp.lds;
      q.fits = true;
      int* ctr = static_cast<int*>(g.ws);
      int* part = reinterpret_cast<int*>(static_cast<char*>(g.ws) + sp.ctr_bytes);
      return sp.X ? launch_s<1, true, OUT, false, true>(g, q, 0, g.M, row_bytes, stream, sp.P,
                                                        ctr, part)
                  : launch_s<1, false, OUT, false, true>(g, q, 0, g.M, row_bytes, stream, sp.P,
                                                         ctr, part);
    }
  }
  // Largest group of activation rows whose staging fits in LDS; one launch per
  // group.
  int64_t mg = g.M;
  while (mg > 1 && !geometry(g.N, row_bytes, mg, accs).fits) mg = (mg + 1) / 2;
  for (int64_t m0 = 0; m0 < g.M; m0 += mg) {
    const int64_t cnt = g.M - m0 < mg ? g.M - m0 : mg;
    const Geometry q = geometry(g.N, row_bytes, cnt, accs);
    if (!q.fits) return hipErrorInvalidValue;
    const hipError_t e = q.X ? launch_x<true, OUT, RES>(g, q, m0, cnt, row_bytes, stream)
                             : launch_x<false, OUT, RES>(g, q, m0, cnt, row_bytes, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Two-plane residual weights: g.N outputs (a multiple of 32), 2 g.N interleaved
// plane rows; fp32 or bf16 output.
hipError_t launch_gemv_mfma_residual(const GemmArgs& g, hipStream_t stream) {
  if (g.N % 32 != 0) return hipErrorInvalidValue;
  switch (g.y_dt) {
    case Elt::F32:
      return launch_out<(int)Elt::F32, true>(g, stream);
    case Elt::BF16:
      return launch_out<(int)Elt::BF16, true>(g, stream);
    default:
      return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Workspace of the allocation-free decode entry point (bwta_gemv_noalloc): one
// file-scope array per GPU, large enough for every cross-block split plan
// (the fixed counter region plus kMaxSplitTiles partial tiles).  Host code never
// passes `scratch` itself to a kernel: it is a host-side stand-in, and the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked up
// once per device with that device current.
constexpr size_t kScratchBytes = kCtrBytes + (size_t)kMaxSplitTiles * 1024;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
bool g_scratch_done[kMaxDevices];

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_workspace(void** ptr, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_done[dev]) {
    // First call on this device (which is current): the device address of its
    // copy of the array, then one clear of the counter region on the caller's
    // stream (a kernel, not a memset, so that the call may be captured in a
    // graph).  Every later call finds the counters zero: each launch returns
    // the ones it used to zero before it ends.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
      const int words = (int)(kCtrBytes / 4);
      hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                         stream, static_cast<uint32_t*>(p), words);
      e = hipGetLastError();
    }
    g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = e;
    g_scratch_done[dev] = true;
  }
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

size_t gemv_mfma_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const Split sp = split_plan(M, N, (K + 63) / 64 * 8);
  return sp.use ? sp.ws_bytes : 0;
}

hipError_t launch_gemv_fused(const GemmArgs& g, const void* X, Elt x_dt, int64_t ldx,
                             uint8_t* o_mask, uint8_t* o_sign, float* o_alpha, int32_t* o_nnz,
                             hipStream_t stream) {
  const FusedIO io{X, ldx, (int)g.K, o_mask, o_sign, o_alpha, o_nnz};
  const bool bf = x_dt == Elt::BF16;
  switch (g.y_dt) {
    case Elt::F32:
      return bf ? launch_fused<(int)Elt::F32, 2>(g, io, stream) : launch_fused<(int)Elt::F32, 1>(g, io, stream);
    case Elt::BF16:
      return bf ? launch_fused<(int)Elt::BF16, 2>(g, io, stream) : launch_fused<(int)Elt::BF16, 1>(g, io, stream);
    case Elt::I32:
      return bf ? launch_fused<(int)Elt::I32, 2>(g, io, stream) : launch_fused<(int)Elt::I32, 1>(g, io, stream);
  }
  return hipErrorInvalidValue;
}

// Workspace of the ternarize-once decode: the decode kernel's own region (split
// counters and partial tiles; none for shapes that never split), whose counter
// region (zero between calls, the same for every shape) ends with the row
// flags, then the exchange planes and scales.  The flags sit at the same offset
// for every shape, inside a region no call leaves non-zero, so calls of any
// shapes can share one workspace.
struct XPLayout {
  size_t split, flags, mask, sign, alpha, nnz, total;
};

XPLayout xp_layout(int64_t M, int64_t N, int64_t K) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t plane = (size_t)M * (size_t)((K + 63) / 64 * 8);
  XPLayout l;
  l.split = gemv_mfma_workspace_bytes(M, N, K);
  l.flags = kCtrBytes - kFlagBytes;
  l.mask = up(l.split > kCtrBytes ? l.split : kCtrBytes);
  l.sign = l.mask + up(plane);
  l.alpha = l.sign + up(plane);
  l.nnz = l.alpha + up((size_t)M * 4);
  l.total = l.nnz + up((size_t)M * 4);
  return l;
}

size_t gemv_fused_xp_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || M > 16) return 0;
  return xp_layout(M, N, K).total;
}

hipError_t launch_gemv_fused_xp(const GemmArgs& g, const void* X, Elt x_dt, int64_t ldx,
                                uint8_t* o_mask, uint8_t* o_sign, float* o_alpha,
                                int32_t* o_nnz, void* ws, size_t ws_bytes, int spin,
                                hipStream_t stream) {
  if (g.M < 1 || g.M > 16 || !ws) return hipErrorNotSupported;
  const XPLayout l = xp_layout(g.M, g.N, g.K);
  if (ws_bytes < l.total || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return hipErrorNotSupported;
  char* base = static_cast<char*>(ws);
  uint8_t* ex_mask = reinterpret_cast<uint8_t*>(base + l.mask);
  uint8_t* ex_sign = reinterpret_cast<uint8_t*>(base + l.sign);
  float* ex_alpha = reinterpret_cast<float*>(base + l.alpha);
  int32_t* ex_nnz = reinterpret_cast<int32_t*>(base + l.nnz);
  GemmArgs g2 = g;
  g2.ws = l.split ? ws : nullptr;
  g2.ws_bytes = l.split;
  const FusedIO io{X, ldx, (int)g.K, o_mask, o_sign, o_alpha, o_nnz,
                   reinterpret_cast<int*>(base + l.flags), spin < 0 ? 0 : spin,
                   ex_mask, ex_sign, ex_alpha, ex_nnz, 1};
  const bool bf = x_dt == Elt::BF16;
  switch (g.y_dt) {
    case Elt::F32:
      return bf ? launch_xp<(int)Elt::F32, 2>(g2, io, stream) : launch_xp<(int)Elt::F32, 1>(g2, io, stream);
    case Elt::BF16:
      return bf ? launch_xp<(int)Elt::BF16, 2>(g2, io, stream) : launch_xp<(int)Elt::BF16, 1>(g2, io, stream);
    case Elt::I32:
      return bf ? launch_xp<(int)Elt::I32, 2>(g2, io, stream) : launch_xp<(int)Elt::I32, 1>(g2, io, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_mfma(const GemmArgs& g, hipStream_t stream) {
  switch (g.y_dt) {
    case Elt::F32:
      return launch_out<(int)Elt::F32>(g, stream);
    case Elt::BF16:
      return launch_out<(int)Elt::BF16>(g, stream);
    case Elt::I32:
      return launch_out<(int)Elt::I32>(g, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace bwta
