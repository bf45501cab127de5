// attention.hip - fused attention over ternary Q and K and binary V^T: for
// every head and query row
//   S[j]   = sum_d t_q[d] t_k[j, d]                     (exact integers)
//   P      = softmax_j(alpha_q alpha_k[j] S[j] * scale)  (fp32 on the GPU)
//   t_p, alpha_p, nnz_p = ternarize(P)                  (the library's rule)
//   O[c]   = (sum_j t_p[j] s_v[c, j]) * (alpha_p alpha_v[c])
// in one launch: the score row never leaves registers and P never reaches
// memory (unless the caller asks for it).
//
// BWTA page ("BWTA: Accurate and Efficient Binarized Transformer by
// Algorithm-Hardware Co-design"), Abstract and "Core claim": the binary /
// ternary MatMul serves the attention operators as well as the linear layers,
// so both attention products take ternarized operands (Q, K, P) and a
// binarized V.  The softmax between them is ordinary fp32 arithmetic; the
// ternarization of P follows the library's rule exactly (pairwise tree sums,
// threshold 0.5 * mean |p|, mean of the kept values), on the P values this
// kernel computed.
//
// Design (head dim 128, L = 256 W keys per head, W in {2, 4, 8}):
// * One block = 64 query rows of one head in 4 passes of 16, W waves.  The
//   head's K planes (32 bytes per key) are staged in LDS once per block with
//   coalesced loads, already merged into the slice scheme's q01/q23 words, so
//   each K byte leaves L2 once per 64 query rows.
// * In a pass, wave w owns the keys [256 w, 256 (w+1)).  Its score tile t
//   (t < 16) holds, in MFMA column c, key 256 w + 16 c + t, so the 16 scores a
//   lane holds per row are consecutive keys: the first four levels of the
//   pairwise tree over the row are register adds, the next four are DPP
//   exchanges within a 16-lane row, the last log2(W) cross the waves through
//   LDS; and a lane's 16 mask bits are half a word of the packed P row.
// * Q K^T on v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 (e2m1) operands, one
//   instruction per 16 x 16 tile: lane group g of both operands holds bit
//   slice g of the 128 values (nibble j of register x <- bit 4j + g of word x,
//   as +-1.0 = 0x2 / 0xA or 0), a permutation of d that A and B share, so the
//   instruction sums t_q[d] t_k[d] over all 128 d exactly.
// * Softmax: u = S * alpha_k[j] per score; with a = alpha_q * scale * log2(e)
//   per row, each wave takes e = exp2(a u - a m_w) against its own maximum m_w
//   (one fma and v_exp_f32) and its sum s_w; one LDS exchange gives the row
//   maximum m and s = sum_w s_w f_w, f_w = exp2(a m_w - a m), and
//   p = e * (f_w / s).
// * P V on the same instruction with the decode kernel's scheme: V^T bits are
//   the A operand (b * {0.5, 1, 2, 2} in slices e = 0..3, brought to b by the
//   A scale 2^{1, 0, -1, -1}), P's mask bits (kept from LDS) the B operand as
//   e2m1 1.0; the products give U = sum t_p b, and O = (nnz_p - 2U) * scales.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bwta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;  // one MFMA k-step of 128 FP4 values
constexpr int kRows = 16;      // query rows per block
constexpr int T = 16;          // score tiles (of 16 keys) per wave
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v4f mfma_fp4(v4i a, v4i b, v4f c, int scale_a) {
  const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
  const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, scale_a, 0, 127);
}

// Bit slice e (0..3) of a ternary (mask, sign) word pair as e2m1: nibble j is
// t at bit 4j + e, with the mask bit moved to nibble bit 1 and the sign bit
// to nibble bit 3.  Rotations keep it one instruction per word for any e.
__device__ __forceinline__ uint32_t ternary_slice(uint32_t m, uint32_t s, int e) {
  const uint32_t mm = __builtin_rotateright32(m, (uint32_t)(e + 31) & 31u);
  const uint32_t ss = __builtin_rotateright32(s, (uint32_t)(e + 29) & 31u);
  return (mm & 0x22222222u) | (ss & 0x88888888u);
}

// Slice e of a binary plane word as the A operand of P V: b * {0.5, 1, 2, 2}.
template <int E>
__device__ __forceinline__ v4i binary_slice(v4u w) {
  v4i o;
#pragma unroll
  for (int x = 0; x < 4; ++x)
    o[x] = (int)(E == 3 ? (w[x] >> 1) & 0x44444444u : w[x] & (0x11111111u << E));
  return o;
}
__device__ __forceinline__ constexpr int binary_scale(int e) { return e == 0 ? 128 : e == 1 ? 127 : 126; }

// Slice e of a 0/1 plane word as e2m1 1.0 (nibble bit 1).
template <int E>
__device__ __forceinline__ v4i unit_slice(v4u m) {
  v4i o;
#pragma unroll
  for (int x = 0; x < 4; ++x) o[x] = (int)(__builtin_rotateright32(m[x], (E + 31) & 31) & 0x22222222u);
  return o;
}

// Reductions over the 16 lanes of a row with DPP moves: lane bit 0
// (quad_perm 1,0,3,2), bit 1 (quad_perm 2,3,0,1), then the mirrors within 8 and
// 16 lanes, which after the first two steps pair the quads 0-1, 2-3 and then
// the halves.  So the sums follow the pairwise tree over the 16 lanes in lane
// order, and every lane of the row ends with the same bits (IEEE addition is
// commutative).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

__device__ __forceinline__ float row_tree(float v) {
  v = v + dppf<kXor1>(v);
  v = v + dppf<kXor2>(v);
  v = v + dppf<kHalfMirror>(v);
  return v + dppf<kMirror>(v);
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dppf<kXor1>(v));
  v = fmaxf(v, dppf<kXor2>(v));
  v = fmaxf(v, dppf<kHalfMirror>(v));
  return fmaxf(v, dppf<kMirror>(v));
}
__device__ __forceinline__ int row_sum_int(int v) {
  v += dpp<kXor1>(v);
  v += dpp<kXor2>(v);
  v += dpp<kHalfMirror>(v);
  return v + dpp<kMirror>(v);
}

// Orders LDS traffic only (no wait on outstanding global loads).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pairwise tree over W (power of two) per-wave partials of row `row`.
template <int W>
__device__ __forceinline__ float wave_tree_lds(const float (*v)[kRows], int row) {
  float t[W];
#pragma unroll
  for (int i = 0; i < W; ++i) t[i] = v[i][row];
  return lane_tree<W>(t);
}

// Slot (16 bytes) of key j (within its head) in the staged K planes: one slot
// of padding after every 16 keys, so the keys 16 c + t (c = 0..7) that one
// read instruction takes for tile t fall in 8 different bank groups, and each
// lane's 16 keys stay contiguous (one base address, immediate offsets).
constexpr int kSlots(int L) { return L + L / 16; }
__device__ __forceinline__ int kslot(int j) { return j + (j >> 4); }

template <int W, int NP, int OUT>
__global__ void __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(4)))
attention_kernel(const uint8_t* __restrict__ q_mask, const uint8_t* __restrict__ q_sign,
                 const float* __restrict__ q_alpha, const uint8_t* __restrict__ k_mask,
                 const uint8_t* __restrict__ k_sign, const float* __restrict__ k_alpha,
                 const uint8_t* __restrict__ v_sign, const float* __restrict__ v_alpha, float scale,
                 void* __restrict__ O, float* __restrict__ p_out, uint8_t* __restrict__ p_mask,
                 float* __restrict__ p_alpha, int32_t* __restrict__ p_nnz) {
  constexpr int KW = 16 * T;       // keys per wave
  constexpr int L = W * KW;        // keys per head
  constexpr int RB = L / 8;        // bytes per packed P row and per V^T row
  constexpr int LPW = 32 / T;      // lanes per 32-bit word of a P row
  __shared__ float red[4][W][kRows];
  __shared__ int red_n[W][kRows];
  // P rows padded by 16 bytes so that the 16 rows read together hit different banks
  __shared__ __attribute__((aligned(16))) uint32_t plane[kRows][RB / 4 + 4];

  // The head's K planes, staged once as q01 words at slot kslot(j) and q23
  // words kSlots(L) slots on.
  extern __shared__ __attribute__((aligned(16))) uint8_t kbuf[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t h = blockIdx.y;
  const int j0 = w * KW + c * T;           // this lane's first key within the head
  const int64_t kk = h * L + j0;

  // 0. Stage K (every thread loads 4 keys' mask and sign rows, coalesced).
  {
    v4u km[L / (W * kWave)], ks[L / (W * kWave)];
#pragma unroll
    for (int i = 0; i < L / (W * kWave); ++i) {
      const int64_t j = (int64_t)i * W * kWave + threadIdx.x;
      km[i] = *reinterpret_cast<const v4u*>(k_mask + (h * L + j) * 16);
      ks[i] = *reinterpret_cast<const v4u*>(k_sign + (h * L + j) * 16);
    }
    // Staged as q01 = (mask bits 4j, 4j+1 | sign bits of the same k, shifted 2)
    // and q23 (the same for 4j+2, 4j+3): slice e of a word is then one mask (odd
    // e) or a shift and a mask (even e) of q01 or q23, as in ternary_slice.
#pragma unroll
    for (int i = 0; i < L / (W * kWave); ++i) {
      const int j = kslot(i * W * kWave + threadIdx.x);
      v4u q01, q23;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        q01[x] = (km[i][x] & 0x33333333u) | ((ks[i][x] << 2) & 0xCCCCCCCCu);
        q23[x] = ((km[i][x] >> 2) & 0x33333333u) | (ks[i][x] & 0xCCCCCCCCu);
      }
      *reinterpret_cast<v4u*>(kbuf + j * 16) = q01;
      *reinterpret_cast<v4u*>(kbuf + (kSlots(L) + j) * 16) = q23;
    }
  }
  lds_barrier();

#pragma unroll 1
  for (int pass = 0; pass < NP; ++pass) {
  const int64_t q0 = h * L + ((int64_t)blockIdx.x * NP + pass) * kRows;  // first query row
  // alpha_k of the lane's keys, reloaded per pass (cache hits) rather than held
  // in registers through the softmax and P V of the previous pass
  const float* kap = k_alpha + kk;
  asm volatile("" : "+v"(kap));
  float ak[T];
#pragma unroll
  for (int t = 0; t < T; t += 4) {
    const v4f v = *reinterpret_cast<const v4f*>(kap + t);
#pragma unroll
    for (int i = 0; i < 4; ++i) ak[t + i] = v[i];
  }

  // 1. Scores.  A = the 16 query rows (lane row c, slice g), B = 16 keys.
  v4i a;
  {
    const v4u m = *reinterpret_cast<const v4u*>(q_mask + (q0 + c) * 16);
    const v4u s = *reinterpret_cast<const v4u*>(q_sign + (q0 + c) * 16);
#pragma unroll
    for (int x = 0; x < 4; ++x) a[x] = (int)ternary_slice(m[x], s[x], g);
  }
  const v4f aq = *reinterpret_cast<const v4f*>(q_alpha + q0 + 4 * g);
  float u[T][4];  // u = S * alpha_k, rows 4g + r of the block, key kk + t
  // lane group g reads q01 (g < 2) or q23 and shifts by 1 for even g
  const uint8_t* kq = kbuf + ((g >> 1) * kSlots(L) + kslot(j0)) * 16;
  const uint32_t ksh = 1u - (uint32_t)(g & 1);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const v4u q = *reinterpret_cast<const v4u*>(kq + t * 16);
    v4i b;
#pragma unroll
    for (int x = 0; x < 4; ++x) b[x] = (int)((q[x] << ksh) & 0xAAAAAAAAu);
    const v4f acc = mfma_fp4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 127);
#pragma unroll
    for (int r = 0; r < 4; ++r) u[t][r] = acc[r] * ak[t];
    // keep the LDS reads of later tiles from being hoisted (registers)
    if ((t & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }

  // 2. Softmax over the row's L keys.  Each wave exponentiates against its own
  // maximum m_w; one exchange gives the row maximum m and the sum
  // s = sum_w s_w f_w with f_w = exp2(a m_w - a m), and p = e * (f_w / s).
  float coef[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    coef[r] = (aq[r] * scale) * kLog2e;
    float v = u[0][r];
#pragma unroll
    for (int t = 1; t < T; ++t) v = fmaxf(v, u[t][r]);
    const float mw = row_max(v);
    const float off = -(coef[r] * mw);
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      u[t][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(coef[r], u[t][r], off));
      sum += u[t][r];
    }
    sum = row_tree(sum);
    if (c == 0) {
      red[0][w][4 * g + r] = mw;
      red[1][w][4 * g + r] = sum;
    }
  }
  lds_barrier();
  // p, then the tree sum of p for mu.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * g + r;
    // Lane c takes wave c % W: the row maximum, then f and s f of that wave, and
    // the pairwise tree over the W waves in order (lane bits 0, 1, then the
    // half-row mirror, which pairs lane quads 0-3 and 4-7).
    const float mi = red[0][c & (W - 1)][row];
    float m = fmaxf(mi, dppf<kXor1>(mi));
    if constexpr (W > 2) m = fmaxf(m, dppf<kXor2>(m));
    if constexpr (W > 4) m = fmaxf(m, dppf<kHalfMirror>(m));
    const float off = -(coef[r] * m);
    float sw = red[1][c & (W - 1)][row] *
               __builtin_amdgcn_exp2f(__builtin_fmaf(coef[r], mi, off));
    sw = sw + dppf<kXor1>(sw);
    if constexpr (W > 2) sw = sw + dppf<kXor2>(sw);
    if constexpr (W > 4) sw = sw + dppf<kHalfMirror>(sw);
    const float fw = __builtin_amdgcn_exp2f(__builtin_fmaf(coef[r], red[0][w][row], off));
    const float k = fw / sw;
    float pr[T];
#pragma unroll
    for (int t = 0; t < T; ++t) pr[t] = u[t][r] = u[t][r] * k;
    const float part = row_tree(lane_tree<T>(pr));
    if (c == 0) red[2][w][row] = part;
  }
  lds_barrier();

  // 3. Ternarize each row: thr = 0.5 * tree(p) / L; keep p > thr.
  uint32_t word[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mu = wave_tree_lds<W>(red[2], 4 * g + r) / (float)L;
    const float thr = 0.5f * mu;
    uint32_t bits = 0;
    float kept[T];
#pragma unroll
    for (int t = T - 1; t >= 0; --t) {
      const float d = thr - u[t][r];  // negative exactly when p > thr
      bits = (bits << 1) | (__float_as_uint(d) >> 31);
      kept[t] = d < 0.f ? u[t][r] : 0.f;
    }
    word[r] = bits;
    const int cnt = row_sum_int(__popc(bits));
    const float part = row_tree(lane_tree<T>(kept));
    if (c == 0) {
      red[3][w][4 * g + r] = part;
      red_n[w][4 * g + r] = cnt;
    }
  }
  // P plane words: the LPW lanes that share a word merge their bits.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t full = word[r] << ((c % LPW) * T);
    full |= (uint32_t)dpp<kXor1>((int)full);
    word[r] = full;
  }
  if (c % LPW == 0) {
    const int wi = (w * KW + c * T) / 32;
#pragma unroll
    for (int r = 0; r < 4; ++r) plane[4 * g + r][wi] = word[r];
    if (p_mask) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<uint32_t*>(p_mask + (q0 + 4 * g + r) * RB + 4 * wi) = word[r];
    }
  }
  if (p_out) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = p_out + (q0 + 4 * g + r) * L + (int64_t)w * KW + c * T;
#pragma unroll
      for (int t = 0; t < T; t += 4)
        *reinterpret_cast<v4f*>(dst + t) = v4f{u[t][r], u[t + 1][r], u[t + 2][r], u[t + 3][r]};
    }
  }
  lds_barrier();
  // alpha_p and nnz_p of query row c (every lane computes its own row's).
  int nz = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) nz += red_n[i][c];
  const float al = nz ? wave_tree_lds<W>(red[3], c) / (float)nz : 0.0f;
  if (w == 0 && g == 0) {
    if (p_alpha) p_alpha[q0 + c] = al;
    if (p_nnz) p_nnz[q0 + c] = nz;
  }

  // 4. O = P V.  Wave w: channel tiles NT w .. NT w + NT - 1, all L keys.
  constexpr int NCH = L / 512;          // 64-byte chunks per row
  constexpr int NT = kHeadDim / 16 / W;  // channel tiles per wave
  v4f acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint8_t* vrow = v_sign + (h * kHeadDim + (NT * w) * 16 + c) * (int64_t)RB + 16 * g;
  // V^T is the same for every pass; reloading it (from L2) per pass is cheaper
  // than keeping it in registers across the passes.
  asm volatile("" : "+v"(vrow));
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const v4u pm = *reinterpret_cast<const v4u*>(&plane[c][16 * ch + 4 * g]);
    const v4i b0 = unit_slice<0>(pm), b1 = unit_slice<1>(pm), b2 = unit_slice<2>(pm),
              b3 = unit_slice<3>(pm);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const v4u vw = *reinterpret_cast<const v4u*>(vrow + (int64_t)i * 16 * RB + 64 * ch);
      acc[i] = mfma_fp4(binary_slice<0>(vw), b0, acc[i], binary_scale(0));
      acc[i] = mfma_fp4(binary_slice<1>(vw), b1, acc[i], binary_scale(1));
      acc[i] = mfma_fp4(binary_slice<2>(vw), b2, acc[i], binary_scale(2));
      acc[i] = mfma_fp4(binary_slice<3>(vw), b3, acc[i], binary_scale(3));
    }
  }
  // Lane (g, c): query row c, channels 16 (NT w + i) + 4g + r.
  const float n = (float)nz;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int ch0 = (NT * w + i) * 16 + 4 * g;
    const v4f av = *reinterpret_cast<const v4f*>(v_alpha + h * kHeadDim + ch0);
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = (n - 2.0f * acc[i][r]) * (al * av[r]);
    const int64_t off = (q0 + c) * kHeadDim + ch0;
    if constexpr (OUT == (int)Elt::BF16) {
      const uint32_t lo = f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(O) + off) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<v4f*>(static_cast<float*>(O) + off) = v4f{y[0], y[1], y[2], y[3]};
    }
  }
  }  // pass
}

template <int W, int OUT>
hipError_t launch_t(const AttentionArgs& a, hipStream_t stream) {
  constexpr int L = 256 * W;
  constexpr int NP = 4;                 // 64 query rows per block
  constexpr size_t lds = 2 * kSlots(L) * 16;  // staged K planes
  auto kfn = attention_kernel<W, NP, OUT>;
  const hipError_t e =
      hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, dim3(L / (kRows * NP), (unsigned)a.heads), dim3(W * kWave), lds, stream, a.q_mask, a.q_sign, a.q_alpha, a.k_mask,
                     a.k_sign, a.k_alpha, a.v_sign, a.v_alpha, a.scale, a.O, a.p_out, a.p_mask,
                     a.p_alpha, a.p_nnz);
  return hipGetLastError();
}

template <int OUT>
hipError_t launch_out(const AttentionArgs& a, hipStream_t stream) {
  switch (a.L) {
    case 512: return launch_t<2, OUT>(a, stream);
    case 1024: return launch_t<4, OUT>(a, stream);
    default: return launch_t<8, OUT>(a, stream);
  }
}

}  // namespace

hipError_t launch_attention(const AttentionArgs& a, hipStream_t stream) {
  if (a.heads <= 0) return hipSuccess;
  if (a.D != kHeadDim || (a.L != 512 && a.L != 1024 && a.L != 2048) || a.heads > 65535)
    return hipErrorInvalidValue;
  return a.o_dt == Elt::BF16 ? launch_out<(int)Elt::BF16>(a, stream)
                             : launch_out<(int)Elt::F32>(a, stream);
}

}  // namespace bwta
