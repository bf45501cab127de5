// probe.hip - measurement kernels of libbwta_probe.so (declared in
// bwta_probe.h): a read-only HBM stream and matrix-core loops, timed by the
// benchmark to measure the chip's ceilings beside the datasheet figures.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bwta_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 16-byte non-temporal loads: a wave reads kPer consecutive 1 KiB chunks (one
// chunk per load instruction, lane l at byte 16 l of the chunk), all issued
// before any is used, then moves on by the grid's span of chunks.
constexpr int kPer = 8;

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf,
                                                          size_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[256];
  const int lane = threadIdx.x & 63;
  const size_t nchunks = (n16 + 63) / 64;
  const size_t wave = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
  const size_t span = (size_t)gridDim.x * 4 * kPer;  // chunks per round of the grid
  uint32_t x = 0;
  for (size_t c0 = wave * kPer; c0 < nchunks; c0 += span) {
    u32x4 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const size_t i = (c0 + j) * 64 + lane;
      v[j] = i < n16 ? __builtin_nontemporal_load(buf + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int t = 0; t < 256; ++t) s ^= red[t];
    sink[blockIdx.x] = s;
  }
}

// 16 independent accumulators per wave (256 of them live in the AGPRs), the
// same operands every round; one wave per SIMD.
template <int FMT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_loop_kernel(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + threadIdx.x / 64;
  v4i a = v4i{0x22222222 ^ lane, 0x2A2A2A2A, 0x22A222A2, 0x2222AAAA ^ wave};
  v4i b = v4i{0x2A22A22A, 0x22222222 ^ lane, 0x2AAA2222, 0x222A2A22};
  uint32_t out = 0;
  if constexpr (FMT == 0) {
    v16f acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
    const v8i a8 = __builtin_shufflevector(a, a, 0, 1, 2, 3, -1, -1, -1, -1);
    const v8i b8 = __builtin_shufflevector(b, b, 0, 1, 2, 3, -1, -1, -1, -1);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[j], 4, 4, 0, 127, 0,
                                                                  127);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) out ^= __float_as_uint(acc[j][lane & 15]);
  } else {
    v16i acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][q] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) out ^= (uint32_t)acc[j][lane & 15];
  }
  // one word per wave (lane 0 of the wave's XOR over its lanes is enough to keep
  // the products live)
  for (int o = 32; o > 0; o >>= 1) out ^= __shfl_xor(out, o, 64);
  if (lane == 0) sink[wave] = out;
}

}  // namespace

extern "C" int bwta_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                      void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) % 16) != 0 ||
      blocks < 0)
    return -1;
  if (blocks == 0) {  // one round of kPer chunks per wave, at most 8192 blocks
    const size_t chunks = (bytes / 16 + 63) / 64;
    const size_t need = (chunks + 4 * kPer - 1) / (4 * kPer);
    blocks = need < 1 ? 1 : need > 8192 ? 8192 : (int)need;
  }
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int bwta_probe_mfma(int fmt, int waves, int iters, uint32_t* sink, void* stream) {
  if (!sink || waves <= 0 || waves % 4 != 0 || iters < 0 || (fmt != 0 && fmt != 1)) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (fmt == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3((unsigned)(waves / 4)), dim3(256), 0, st, iters,
                       sink);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3((unsigned)(waves / 4)), dim3(256), 0, st, iters,
                       sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
