// sa_calib.hip -- calibration kernels for the measurements beside the attention path on
// gfx950: a dense bf16 MFMA throughput loop (the measured counterpart of the vendor peak)
// and random fixed-size chunk reads from a region of a chosen size (what gathers of K/V
// tiles can get from L2, from the MALL and from HBM).  They compute nothing of the method.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));
constexpr int kCalibThreads = 256;

// four independent accumulator chains per wave keep the MFMA pipe full; operands live
// in registers (no memory traffic); one value per thread is stored so nothing is dropped
__global__ void __launch_bounds__(kCalibThreads) k_calib_mfma(int32_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  cbf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  cf32x16 c0, c1, c2, c3;
#pragma unroll
  for (int v = 0; v < 16; ++v) c0[v] = c1[v] = c2[v] = c3[v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

__device__ inline uint64_t splitmix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

// each workgroup reads `reads` chunks, each at a pseudo-random chunk-aligned offset of the
// region, with 16-byte loads spread over its threads
__global__ void __launch_bounds__(kCalibThreads)
    k_calib_gather(const uint4* buf, int64_t n_chunks, int32_t chunk_vec, int32_t reads, uint64_t seed, float* sink) {
  uint32_t acc = 0;
  for (int r = 0; r < reads; ++r) {
    const uint64_t h = splitmix64(seed ^ ((uint64_t)blockIdx.x << 20) ^ (uint64_t)r);
    const uint4* chunk = buf + (int64_t)(h % (uint64_t)n_chunks) * chunk_vec;
    for (int x = threadIdx.x; x < chunk_vec; x += kCalibThreads) {
      const uint4 u = chunk[x];
      acc ^= u.x ^ u.y ^ u.z ^ u.w;
    }
  }
  sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = (float)(acc & 0xffu);
}

}  // namespace

hipError_t launch_calib_mfma(int32_t n_wg, int32_t iters, float* sink, hipStream_t stream) {
  k_calib_mfma<<<dim3((unsigned)n_wg), dim3(kCalibThreads), 0, stream>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_calib_gather(const void* buf, int64_t region_bytes, int32_t chunk_bytes, int32_t n_wg, int32_t reads,
                               uint64_t seed, float* sink, hipStream_t stream) {
  k_calib_gather<<<dim3((unsigned)n_wg), dim3(kCalibThreads), 0, stream>>>(
      static_cast<const uint4*>(buf), region_bytes / chunk_bytes, chunk_bytes / 16, reads, seed, sink);
  return hipGetLastError();
}

}  // namespace sa
