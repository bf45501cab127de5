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

// Buffer descriptor with range checking over `bytes` (raw buffer: an offset
// at or past `bytes` reads 0).  The base goes through readfirstlane so the
// descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t checked_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

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

// RES: two-plane residual weights (planes interleaved in groups of 32 rows), N
// counts outputs.  The wave of output tile o (16 outputs) streams both of its
// plane tiles - rows 64 (o / 2) + 16 (o % 2) and 32 rows further - with half as
// many chunks per batch (the same bytes in flight), multiplies both by the same
// activation operands, and the epilogue writes
// y = (T - 2 U1) (alpha_a alpha1) + (T - 2 U2) (alpha_a alpha2).
template <int S, bool X, int OUT, bool RES = false>
__global__ void __launch_bounds__(kMaxW * kWave)
gemv_mfma_kernel(const uint8_t* __restrict__ a_mask, const uint8_t* __restrict__ a_sign,
                 const float* __restrict__ a_alpha, int M, const uint8_t* __restrict__ w_sign,
                 const float* __restrict__ w_alpha, int64_t N, int row_bytes,
                 void* __restrict__ Y, int64_t ldy) {
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
  const int64_t ot = (int64_t)blockIdx.x * R + rg;  // output tile
  const int64_t n0 = ot * 16;
  const int64_t p1 = RES ? 64 * (ot >> 1) + 16 * (ot & 1) : n0;  // its (first) plane rows
  const int64_t rows_left = N - n0;
  const int rows_here = rows_left <= 0 ? 0 : (rows_left < 16 ? (int)rows_left : 16);
  const int chunks = (row_bytes + 63) / 64;
  const int c0 = chunks * ks / S;
  const int c1 = chunks * (ks + 1) / S;
  const LdsLayout L = lds_layout(X, chunks, M, S, R, RES ? 2 : 1);
  int* tsum = reinterpret_cast<int*>(smem + L.t_off);

  // 1. Epilogue scales.  Items: S = 1, the lanes of the own wave; S > 1, item
  //    p = threadIdx.x (row group p / 64, lane p % 64) when p < R * 64.
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  const int p_item = S == 1 ? lane : (int)threadIdx.x;
  const bool item_ok = S == 1 || p_item < R * kWave;
  const int64_t nb_item = S == 1 ? n0 : ((int64_t)blockIdx.x * R + p_item / kWave) * 16;
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
    const __amdgpu_buffer_rsrc_t aars = checked_rsrc(a_alpha, (uint32_t)M * 4u);
    aa = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       aars, (int)((l_item & 15) * 4), 0, 0));
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
  const int nsu = (units + (int)blockDim.x - 1) / (int)blockDim.x;  // rounds, uniform
  const __amdgpu_buffer_rsrc_t mrs = checked_rsrc(a_mask, (uint32_t)M * (uint32_t)row_bytes);
  const __amdgpu_buffer_rsrc_t srs = checked_rsrc(a_sign, (uint32_t)M * (uint32_t)row_bytes);
  v4u sm[kMaxSU], ss[kMaxSU];
#pragma unroll
  for (int k = 0; k < kMaxSU; ++k) {
    if (k < nsu) {
      const int u = (int)threadIdx.x + k * (int)blockDim.x;
      int m, c, gg;
      unit_pos(u, m, c, gg);
      const uint32_t off = u < units ? (uint32_t)(m * row_bytes + 64 * c + 16 * gg) : kOOB;
      sm[k] = __builtin_amdgcn_raw_buffer_load_b128(mrs, (int)off, 0, 0);
      ss[k] = __builtin_amdgcn_raw_buffer_load_b128(srs, (int)off, 0, 0);
    }
  }

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
  __builtin_amdgcn_sched_barrier(0);

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
  auto stage_unit = [&](int u, v4u vm, v4u vs) {
    int m, c, gg;
    unit_pos(u, m, c, gg);
    const int valid = row_bytes - 64 * c - 16 * gg;  // bytes of this unit inside the row
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
  for (int u = (int)threadIdx.x + kMaxSU * (int)blockDim.x; u < units; u += (int)blockDim.x) {
    int m, c, gg;
    unit_pos(u, m, c, gg);
    const uint32_t off = (uint32_t)(m * row_bytes + 64 * c + 16 * gg);
    stage_unit(u, __builtin_amdgcn_raw_buffer_load_b128(mrs, (int)off, 0, 0),
               __builtin_amdgcn_raw_buffer_load_b128(srs, (int)off, 0, 0));
  }
  if constexpr (X) {
    for (int z = threadIdx.x; z < 256; z += blockDim.x)  // the extra chunk
      *reinterpret_cast<v4u*>(smem + (uint32_t)chunks * 4096u + z * 16) = v4u{0u, 0u, 0u, 0u};
  } else {
    if (threadIdx.x < 2)
      *reinterpret_cast<v4u*>(smem + L.zero_off + 16 * threadIdx.x) = v4u{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int b = 1; b < kNB; ++b) issue(b, c0 + b * PF);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();

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
        const uint32_t ao = am_base + (uint32_t)c * a_step;
        v4i bop[4];
        if constexpr (X) {
          // lane slot of chunk c (rows m >= M: the cleared extra chunk)
          const uint32_t xo = live ? (uint32_t)c * 4096u +
                                         (uint32_t)(g * 16 + (r ^ (((c & 1) << 2) | g))) * 16u
                                   : (uint32_t)chunks * 4096u;
#pragma unroll
          for (int e = 0; e < 4; ++e) bop[e] = *reinterpret_cast<const v4i*>(smem + xo + e * 1024);
        } else {
          const v4u am = *reinterpret_cast<const v4u*>(smem + ao);
          const v4u as = *reinterpret_cast<const v4u*>(smem + as_base + (uint32_t)c * a_step);
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
  auto store = [&](int l, v4f u4, v4f u4b, int64_t nb) {
    const int m = l & 15;
    const int64_t n = nb + 4 * (l >> 4);
    if (m >= M || n >= N) return;
    int tm = 0;
    for (int w2 = 0; w2 < W; ++w2) tm += tsum[w2 * 16 + m];
    const float t = (float)tm;
    uint32_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float accf = t - 2.0f * u4[u];  // exact: integers below 2^24
      if constexpr (OUT == (int)Elt::I32) {
        o[u] = (uint32_t)(int)accf;
      } else {
        float y = accf * (aa * ab[u]);
        if constexpr (RES) {
          const float y2 = (t - 2.0f * u4b[u]) * (aa * ab2[u]);
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

  if constexpr (S == 1) {
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

template <int S, bool X, int OUT, bool RES = false>
hipError_t launch_s(const GemmArgs& g, const Geometry& q, int64_t m0, int64_t mg,
                    int64_t row_bytes, hipStream_t stream) {
  auto kfn = gemv_mfma_kernel<S, X, OUT, RES>;
  hipError_t e = hipFuncSetAttribute((const void*)kfn,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)q.lds);
  if (e != hipSuccess) return e;
  constexpr int ES = OUT == (int)Elt::BF16 ? 2 : 4;
  hipLaunchKernelGGL(kfn, dim3((unsigned)q.blocks), dim3((unsigned)(q.S * q.R * kWave)), q.lds,
                     stream, g.a_mask + m0 * row_bytes, g.a_sign + m0 * row_bytes,
                     g.a_alpha ? g.a_alpha + m0 : nullptr, (int)mg, g.b_sign, g.b_alpha, g.N,
                     (int)row_bytes, static_cast<char*>(g.Y) + m0 * g.ldy * ES, g.ldy);
  return hipGetLastError();
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
