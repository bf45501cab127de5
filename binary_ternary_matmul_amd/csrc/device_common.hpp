// device_common.hpp - small device helpers shared by the libbwta kernels.
//
// Reductions here follow the library's fixed pairwise-tree order (a perfect
// binary tree over the values zero-padded to a power of two), so every scale
// the kernels compute is bit-identical to that definition regardless of how
// the work is spread over lanes and waves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bwta {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load that bypasses cache retention (data read exactly once).
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The value of lane (lane ^ b) for b a power of two below 64 (b a compile-time
// constant once the caller is unrolled): DPP quad permutes for bits 0 and 1,
// the swizzle unit's xor mode (within 32 lanes) for bits 2 to 4, and a lane
// permute for bit 5.  None needs a per-lane address.
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int b) {
  switch (b) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
    case 4: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);
    case 8: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x201F);
    case 16: return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
    default: return (uint32_t)__builtin_amdgcn_ds_bpermute((__lane_id() ^ b) << 2, (int)v);
  }
}
__device__ __forceinline__ float xor_lane(float v, int b) {
  return __uint_as_float(xor_lane(__float_as_uint(v), b));
}
__device__ __forceinline__ int xor_lane(int v, int b) { return (int)xor_lane((uint32_t)v, b); }

// Buffer descriptor over [base, base + bytes) with range checking: a load at
// or past `bytes` reads 0 and a store there is dropped.  The base goes through
// readfirstlane so that the descriptor lives in SGPRs (the caller's base must
// be wave-uniform).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t checked_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Pairwise tree over N (power of two) values held by one lane.
template <int N>
__device__ __forceinline__ float lane_tree(const float (&v)[N]) {
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = v[i];
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  }
  return t[0];
}

// Tree over N (power of two, <= 64) groups x 64 lanes.  Lane l holds in v[i] the
// partial of group i over its own contiguous run of elements; within a group
// the runs of lanes 0..63 are consecutive, and group i precedes group i+1.
// The result, returned in every lane, is the root of the perfect tree over all
// N*64 runs: lanes are paired by lane bit 0, then bit 1, ... inside each group,
// and groups are then paired 0-1, 2-3, ...
//
// Phase 1 is a reduce-scatter: at step s a lane keeps the half of its groups
// selected by lane bit s and receives the partner's partial of the same
// groups, so after log2(N) steps each lane holds one group, whose index is the
// bit-reversal of the lane's low log2(N) bits.  Phase 2 finishes the lane tree
// of that group over the remaining lane bits.  Phase 3 pairs groups: group
// index bit b sits in lane bit log2(N)-1-b.  IEEE addition is commutative, so
// the partner's operand order does not change the bits.
template <int N>
__device__ __forceinline__ float wave_tree(const float (&in)[N]) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  const int lane = __lane_id();
  float v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = in[i];
  int s = 0;
#pragma unroll
  for (int cnt = N; cnt > 1; cnt >>= 1, ++s) {
    // all-ones when this lane keeps the upper half; the halves are blended
    // bitwise (a select here gets rewritten into a runtime register index)
    const uint32_t hi = 0u - (uint32_t)((lane >> s) & 1);
#pragma unroll
    for (int j = 0; j < cnt / 2; ++j) {
      const uint32_t lo_b = __float_as_uint(v[j]), up_b = __float_as_uint(v[j + cnt / 2]);
      const float keep = __uint_as_float((lo_b & ~hi) | (up_b & hi));
      const float send = __uint_as_float((up_b & ~hi) | (lo_b & hi));
      const float recv = xor_lane(send, 1 << s);
      v[j] = keep + recv;
    }
  }
  float r = v[0];
#pragma unroll
  for (int b = s; b < 6; ++b) r = r + xor_lane(r, 1 << b);
#pragma unroll
  for (int b = s - 1; b >= 0; --b) r = r + xor_lane(r, 1 << b);
  return r;
}

// Exact integer sum over the 64 lanes.
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int b = 0; b < 6; ++b) v += xor_lane(v, 1 << b);
  return v;
}

// Pairwise tree over W (power of two, <= 16) values; zero padding to 16 leaves
// leaves the root unchanged.
__device__ __forceinline__ float tree16(const float* v, int W) {
  float t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) t[i] = i < W ? v[i] : 0.0f;
#pragma unroll
  for (int w = 16; w > 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  }
  return t[0];
}

}  // namespace bwta
