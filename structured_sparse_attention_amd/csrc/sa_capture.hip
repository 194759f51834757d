// sa_capture.hip -- pattern capture and pattern extension on gfx950.
//
// Pith review of "DAM: Dynamic Attention Mask for Long-Context Large Language
// Model Inference Acceleration", "What carries the argument": averaged attention
// maps get a Box-Cox transform with lambda = 0.5 (small values amplified), a
// threshold tau = 0.3 gives the binary true mask M, every diagonal (i, i-r) and
// vertical (i, c), i >= c, of the pattern pool is scored by
// gamma = sum(M * P) / sum(P), and patterns with gamma >= mu = 0.8 are kept; for
// longer inputs the kept patterns are pasted into an S x S mask ("Circularity
// Check" step 1: the extended mask is the union of the matched patterns).
// Referee Report minor comment 1: the stabiliser epsilon is 1e-8 or 1e-10 (a
// parameter here).  The pages do not say how the transformed values are scaled
// before the threshold; they are min-max normalised per causal row (or per map).
//
// Exactness: every step is fp64 with correctly rounded sqrt and division and no
// contraction, so the mask, the hit counts and the keep flags equal those of any
// IEEE fp64 evaluation in the same order.  The transform is monotone
// non-decreasing in A, so the row (or map) minimum and maximum of the transformed
// values are the transforms of the fp32 minimum and maximum of A: the min/max pass
// runs in fp32 and each element is transformed once.
//
// Layout: one 1024-thread workgroup per map; wave w takes rows w, w+16, ...; lanes
// take columns, four loads in flight per lane.  Hits accumulate with LDS atomics; the map is read once from HBM
// (the causal half) plus once more for the fp32 row min/max, which hits in cache.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;  // 16 waves per map: two maps fill a CU's 32 wave slots

__device__ inline double box_cox_half(float a, double eps, double lambda) {
#pragma clang fp contract(off)
  const double x = (double)a + eps;
  const double s = sqrt(x);
  return (s - 1.0) / lambda;
}

__device__ inline float wave_min(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__global__ void __launch_bounds__(kThreads)
    k_capture(const float* maps, int32_t L, double lambda, double eps, double tau, double mu, int32_t norm_scope,
              uint8_t* keep_diag, uint8_t* keep_vert, int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask) {
#pragma clang fp contract(off)
  extern __shared__ int32_t hits[];  // [L] diagonal hits, then [L] vertical hits
  __shared__ float red[2 * (kThreads / 64)];
  int32_t* hd = hits;
  int32_t* hv = hits + L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t map = blockIdx.x;
  const float* A = maps + map * (int64_t)L * L;
  for (int r = tid; r < L; r += kThreads) {
    hd[r] = 0;
    hv[r] = 0;
  }
  float gmin = INFINITY, gmax = -INFINITY;
  if (norm_scope == 1) {
    float mn = INFINITY, mx = -INFINITY;
    for (int i = wave; i < L; i += kThreads / 64)
      for (int j = lane; j <= i; j += 64) {
        const float a = A[(int64_t)i * L + j];
        mn = fminf(mn, a);
        mx = fmaxf(mx, a);
      }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      red[wave] = mn;
      red[kThreads / 64 + wave] = mx;
    }
    __syncthreads();
    for (int w = 0; w < kThreads / 64; ++w) {
      gmin = fminf(gmin, red[w]);
      gmax = fmaxf(gmax, red[kThreads / 64 + w]);
    }
  }
  __syncthreads();

  for (int i = wave; i < L; i += kThreads / 64) {
    const float* row = A + (int64_t)i * L;
    float amin = gmin, amax = gmax;
    if (norm_scope == 0) {
      float mn = INFINITY, mx = -INFINITY;
      for (int jb = 0; jb <= i; jb += 4 * 64) {
        float a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = jb + u * 64 + lane;
          a[u] = j <= i ? row[j] : INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = jb + u * 64 + lane;
          if (j <= i) {
            mn = fminf(mn, a[u]);
            mx = fmaxf(mx, a[u]);
          }
        }
      }
      amin = wave_min(mn);
      amax = wave_max(mx);
    }
    const double ymin = box_cox_half(amin, eps, lambda);
    const double ymax = box_cox_half(amax, eps, lambda);
    const bool flat = (ymax == ymin);
    const double range = ymax - ymin;
    uint8_t* mrow = true_mask ? true_mask + (map * L + i) * (int64_t)L : nullptr;
    for (int jb = 0; jb < L; jb += 4 * 64) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * 64 + lane;
        a[u] = j <= i ? row[j] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * 64 + lane;
        if (j >= L) continue;
        uint8_t keep = 0;
        if (j <= i) {
          const double y = box_cox_half(a[u], eps, lambda);
          keep = flat ? 1 : (((y - ymin) / range) >= tau);
          if (keep) {
            atomicAdd(&hd[i - j], 1);
            atomicAdd(&hv[j], 1);
          }
        }
        if (mrow) mrow[j] = keep;
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < L; r += kThreads) {
    const double size = (double)(L - r);
    keep_diag[map * L + r] = ((double)hd[r] / size) >= mu;
    keep_vert[map * L + r] = ((double)hv[r] / size) >= mu;
    if (diag_hits) diag_hits[map * L + r] = hd[r];
    if (vert_hits) vert_hits[map * L + r] = hv[r];
  }
}

// kept flags -> CSR descriptor lists at length S (entries < S).  One workgroup.
constexpr int kDescThreads = 1024;
__global__ void __launch_bounds__(kDescThreads)
    k_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L, int32_t S,
              int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr, int32_t* vert_col) {
  const int tid = threadIdx.x;
  const int32_t Lc = min(L, S);
  for (int m = tid; m < n_maps; m += kDescThreads) {
    int32_t cd = 0, cv = 0;
    for (int r = 0; r < Lc; ++r) {
      cd += keep_diag[(int64_t)m * L + r] != 0;
      cv += keep_vert[(int64_t)m * L + r] != 0;
    }
    diag_ptr[m + 1] = cd;
    vert_ptr[m + 1] = cv;
  }
  __syncthreads();
  if (tid == 0) {
    diag_ptr[0] = 0;
    vert_ptr[0] = 0;
    for (int m = 0; m < n_maps; ++m) {
      diag_ptr[m + 1] += diag_ptr[m];
      vert_ptr[m + 1] += vert_ptr[m];
    }
  }
  __syncthreads();
  for (int m = tid; m < n_maps; m += kDescThreads) {
    int32_t pd = diag_ptr[m], pv = vert_ptr[m];
    for (int r = 0; r < Lc; ++r) {
      if (keep_diag[(int64_t)m * L + r]) diag_off[pd++] = r;
      if (keep_vert[(int64_t)m * L + r]) vert_col[pv++] = r;
    }
  }
}

}  // namespace

hipError_t launch_capture(const float* maps, int32_t n_maps, int32_t L, double lambda, double eps, double tau,
                          double mu, int32_t norm_scope, uint8_t* keep_diag, uint8_t* keep_vert, int32_t* diag_hits,
                          int32_t* vert_hits, uint8_t* true_mask, hipStream_t stream) {
  const size_t lds = 2 * sizeof(int32_t) * (size_t)L;
  hipLaunchKernelGGL(k_capture, dim3((unsigned)n_maps), dim3(kThreads), lds, stream, maps, L, lambda, eps, tau, mu,
                     norm_scope, keep_diag, keep_vert, diag_hits, vert_hits, true_mask);
  return hipGetLastError();
}

hipError_t launch_patterns_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L,
                                   int32_t S, int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr,
                                   int32_t* vert_col, hipStream_t stream) {
  hipLaunchKernelGGL(k_to_desc, dim3(1), dim3(kDescThreads), 0, stream, keep_diag, keep_vert, n_maps, L, S, diag_ptr,
                     diag_off, vert_ptr, vert_col);
  return hipGetLastError();
}

}  // namespace sa
