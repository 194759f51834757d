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
// Other lambdas (Referee Report major comment 4 asks how the masks move with
// lambda, tau, mu and the capture length) use the textbook Box-Cox form.
//
// Exactness: at lambda = 0.5 every step is fp64 with correctly rounded sqrt and
// division and no contraction, so the mask, the hit counts and the keep flags
// equal those of any IEEE fp64 evaluation in the same order.  Other lambdas go
// through the device pow / log, a few ulp from the correctly rounded value: only
// cells whose normalised score lies within about 1e-15 of tau can differ.  The
// transform is monotone non-decreasing in A for every lambda, so the row (or map)
// minimum and maximum of the transformed values are the transforms of the fp32
// minimum and maximum of A: the min/max pass runs in fp32 and each element is
// transformed once.
//
// At lambda = 0.5 the keep test is also monotone in A (every step rounds monotonically), so each
// row's kept elements are those at or above one fp32 threshold, found per row by bisection with the
// same fp64 steps; the element pass then compares in fp32 and needs no fp64 at all.
//
// Layout: one 1024-thread workgroup per map.  Pass 1: the fp32 min/max of every row (wave w takes rows
// w, w+16, ..., four rows at a time, lanes over columns); pass 2: one thread per row transforms the
// extremes and finds the threshold; pass 3: the element pass (lanes over columns, four loads in
// flight per lane), hits accumulating with LDS atomics.  The causal half of the map is read twice.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 1024;  // 16 waves per map: two maps fill a CU's 32 wave slots

// Box-Cox of x = A + eps: (sqrt(x) - 1) / 0.5 at lambda = 0.5 (correctly rounded, exact),
// log x at lambda = 0, (x^lambda - 1) / lambda otherwise (device pow / log: a few ulp).
enum { kBoxCoxHalf = 0, kBoxCoxLog = 1, kBoxCoxPow = 2 };
template <int KIND>
__device__ inline double box_cox(float a, double eps, double lambda) {
#pragma clang fp contract(off)
  const double x = (double)a + eps;
  if constexpr (KIND == kBoxCoxHalf) {
    const double s = sqrt(x);
    return (s - 1.0) / lambda;
  } else if constexpr (KIND == kBoxCoxLog) {
    return log(x);
  } else {
    return (pow(x, lambda) - 1.0) / lambda;
  }
}

__device__ inline float wave_min(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// How a row's keep flags are decided in the element pass.
enum { kRowThreshold = 0, kRowAll = 1, kRowNone = 2, kRowEach = 3 };

// The keep rule of one causal row from its fp32 extremes (pass 2 below explains why a threshold is
// exact): mode, and for kRowThreshold the smallest float that passes.  At lambda = 0.5 the search
// starts from the inverse of the transform, a = (1 + (ymin + tau * range) / 2)^2 - eps, which is a
// few fp64 roundings from the answer: a short walk over neighbouring floats settles it, and a
// bisection over what is left covers any start that is further off.  The answer does not depend on
// the start: it is the unique smallest passing value of a monotone test.
template <int KIND>
__device__ inline void row_rule(float amin, float amax, double eps, double lambda, double tau, int& mode,
                                float& thr) {
#pragma clang fp contract(off)
  const double ymin = box_cox<KIND>(amin, eps, lambda);
  const double ymax = box_cox<KIND>(amax, eps, lambda);
  mode = kRowEach;
  thr = 0.0f;
  if (ymax == ymin) {
    mode = 1.0 >= tau ? kRowAll : kRowNone;  // flat: t = 1 for every element
    return;
  }
  if (!(amin >= 0.0f && amax < INFINITY)) return;
  const double range = ymax - ymin;
  auto pass = [&](uint32_t bits) { return (box_cox<KIND>(__uint_as_float(bits), eps, lambda) - ymin) / range >= tau; };
  const uint32_t bmin = __float_as_uint(amin) & 0x7fffffffu, bmax = __float_as_uint(amax);
  if (!pass(bmax)) {
    mode = kRowNone;
    return;
  }
  mode = kRowThreshold;
  uint32_t lo = bmin, hi = bmax;  // the answer lies in [lo, hi], and hi passes
  if constexpr (KIND == kBoxCoxHalf) {
    const double sr = 1.0 + 0.5 * (ymin + tau * range);
    const double a = sr > 0.0 ? sr * sr - eps : 0.0;
    const uint32_t c = a <= (double)amin ? bmin : a >= (double)amax ? bmax : __float_as_uint((float)a);
    if (pass(c)) {
      hi = c;
      for (int k = 0; k < 8 && hi > lo; ++k) {
        if (!pass(hi - 1)) {
          lo = hi;  // hi passes and the float below it does not
          break;
        }
        --hi;
      }
    } else {
      lo = c + 1;  // c < bmax here, since bmax passes
      for (int k = 0; k < 8 && lo < hi; ++k) {
        if (pass(lo)) {
          hi = lo;  // everything below lo failed
          break;
        }
        ++lo;
      }
    }
  }
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (pass(mid)) hi = mid;
    else lo = mid + 1;
  }
  thr = __uint_as_float(lo);
}

template <int KIND>
__global__ void __launch_bounds__(kThreads)
    k_capture(const float* maps, int32_t L, double lambda, double eps, double tau, double mu, int32_t norm_scope,
              uint8_t* keep_diag, uint8_t* keep_vert, int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask) {
#pragma clang fp contract(off)
  // LDS: [L] diagonal hits, [L] vertical hits, then per row: A min, A max, threshold, mode
  extern __shared__ int32_t lds[];
  __shared__ float red[2 * (kThreads / 64)];
  int32_t* hd = lds;
  int32_t* hv = lds + L;
  float* rmin = reinterpret_cast<float*>(lds + 2 * L);
  float* rmax = reinterpret_cast<float*>(lds + 3 * L);
  float* rthr = reinterpret_cast<float*>(lds + 4 * L);
  int32_t* rmode = lds + 5 * L;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t map = blockIdx.x;
  const float* A = maps + map * (int64_t)L * L;
  for (int r = tid; r < L; r += kThreads) {
    hd[r] = 0;
    hv[r] = 0;
  }

  // 1. the fp32 minimum and maximum of every causal row (norm_scope 0) or of the map (1)
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
    float gmin = INFINITY, gmax = -INFINITY;
    for (int w = 0; w < kThreads / 64; ++w) {
      gmin = fminf(gmin, red[w]);
      gmax = fmaxf(gmax, red[kThreads / 64 + w]);
    }
    for (int r = tid; r < L; r += kThreads) {
      rmin[r] = gmin;
      rmax[r] = gmax;
    }
  } else {
    // four rows per wave at a time (rows w, w + 16, w + 32, w + 48 of each block of 64), so that four
    // independent loads and reductions are in flight
    constexpr int kRows = 4, kStride = kThreads / 64;
    for (int i0 = wave; i0 < L; i0 += kRows * kStride) {
      float mn[kRows], mx[kRows];
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        mn[q] = INFINITY;
        mx[q] = -INFINITY;
      }
      const int ilast = min(L - 1, i0 + (kRows - 1) * kStride);
      for (int j = lane; j <= ilast; j += 64) {
        float a[kRows];
#pragma unroll
        for (int q = 0; q < kRows; ++q) {
          const int i = i0 + q * kStride;
          a[q] = (i < L && j <= i) ? A[(int64_t)i * L + j] : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < kRows; ++q) {
          const int i = i0 + q * kStride;
          if (i < L && j <= i) {
            mn[q] = fminf(mn[q], a[q]);
            mx[q] = fmaxf(mx[q], a[q]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kRows; ++q) {
        const int i = i0 + q * kStride;
        const float lo = wave_min(mn[q]), hi = wave_max(mx[q]);
        if (lane == 0 && i < L) {
          rmin[i] = lo;
          rmax[i] = hi;
        }
      }
    }
  }
  __syncthreads();

  // 2. one thread per row: the transform of the extremes and the keep threshold.  At lambda = 0.5 the
  // test t >= tau, t = (y(a) - ymin) / (ymax - ymin), is monotone non-decreasing in a: each step
  // (a + eps, the correctly rounded sqrt, - 1, * 2, - ymin, / range) rounds monotonically.  So for
  // finite a >= 0 the kept elements of a row are those at or above the smallest float that passes,
  // found by bisection over the ordered bit patterns of [min, max] with the same fp64 steps.  Box-Cox
  // is increasing for every lambda; with the device log / pow (a few ulp, not guaranteed monotone at
  // that scale) the threshold decides like a per-element test except for cells whose t lies within a
  // few ulp of tau, the cells that may differ from a correctly rounded evaluation anyway.  Rows with
  // a negative or non-finite extreme test each element.
  for (int r = tid; r < L; r += kThreads) {
    int mode;
    float thr;
    row_rule<KIND>(rmin[r], rmax[r], eps, lambda, tau, mode, thr);
    rmode[r] = mode;
    rthr[r] = thr;
  }
  __syncthreads();

  // 3. element pass: keep flags, hits, optional true mask
  for (int i = wave; i < L; i += kThreads / 64) {
    const float* row = A + (int64_t)i * L;
    const int mode = rmode[i];
    const float thr = rthr[i];
    double ymin = 0.0, range = 1.0;
    if (mode == kRowEach) {
      ymin = box_cox<KIND>(rmin[i], eps, lambda);
      range = box_cox<KIND>(rmax[i], eps, lambda) - ymin;
    }
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
          if (mode == kRowThreshold) keep = a[u] >= thr;
          else if (mode == kRowAll) keep = 1;
          else if (mode == kRowEach) keep = (box_cox<KIND>(a[u], eps, lambda) - ymin) / range >= tau;
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

// ---------------------------------------------------------------------------
// One read of the map: the same keep flags and hits as k_capture for lambda = 0.5, per-row
// extremes (norm_scope 0) and L <= 512 with L % 4 == 0 (the capture length of the pages is 512).
// 512 threads per map (about 100 VGPRs, so two maps share a CU).  A wave holds kRowBatch consecutive
// causal rows in registers (lane l: columns 4(l + 64u) .. +3), reduces each row's extremes across the
// wave, lets lane q find row q's rule (row_rule, all rows of the batch at once), and counts hits from
// the same registers: diagonal hits with LDS atomics, vertical hits in registers (the lane's columns
// are fixed) added to LDS once at the end.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 512, kRowBatch = 2, kRowMaxL = 512;

__global__ void __launch_bounds__(kRowThreads)
    k_capture_rows(const float* maps, int32_t L, double eps, double tau, double mu, uint8_t* keep_diag,
                   uint8_t* keep_vert, int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask) {
#pragma clang fp contract(off)
  constexpr int NU = kRowMaxL / 256;  // float4 chunks per lane and row
  constexpr int NW = kRowThreads / 64;
  constexpr int kDiag = kRowBatch + 3;  // diagonals of one chunk's cells in a batch
  static_assert(kRowMaxL / NW <= 255, "a lane's vertical hits per column fit a byte");
  __shared__ int32_t hd[kRowMaxL + 64], hv[kRowMaxL];  // hd[kRowMaxL + lane]: a sink for zero adds
  // the wave index is uniform (a scalar register), so that row indices and row predicates are scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t map = blockIdx.x;
  const float* A = maps + map * (int64_t)L * L;
  const int nq = L / 4;  // float4 per row
  const uint32_t map_bytes = (uint32_t)L * L * 4u;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, map_bytes, 0x00020000);
  for (int r = tid; r < kRowMaxL + 64; r += kRowThreads) hd[r] = 0;
  for (int r = tid; r < kRowMaxL; r += kRowThreads) hv[r] = 0;
  __syncthreads();
  // vertical hits of this lane's columns, one byte per column (a lane sees at most L / NW <= 64 rows)
  uint32_t vh[NU] = {};
  // a batch's causal cells; cells past the row, the map or the rows read as zero (buffer range)
  auto load_batch = [&](int i0, float4 (&dst)[kRowBatch][NU]) {
#pragma unroll
    for (int q = 0; q < kRowBatch; ++q)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = lane + 64 * u, i = i0 + q;
        const uint32_t off = (i < L && c < nq && 4 * c <= i) ? (uint32_t)(i * L + 4 * c) * 4u : map_bytes;
        dst[q][u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rsA, off, 0, 0));
      }
  };
  // the next batch's loads are in flight while this one is reduced, ruled and counted
  float4 a[kRowBatch][NU], an[kRowBatch][NU];
  load_batch(kRowBatch * wave, a);
  for (int i0 = kRowBatch * wave; i0 < L; i0 += kRowBatch * NW) {
    load_batch(i0 + kRowBatch * NW, an);
    // extremes of each causal row
    float mn[kRowBatch], mx[kRowBatch];
#pragma unroll
    for (int q = 0; q < kRowBatch; ++q) {
      mn[q] = INFINITY;
      mx[q] = -INFINITY;
      const int i = i0 + q;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = lane + 64 * u;
        // a chunk with a cell in the row starts in the row; its cells past the row repeat its first
        // cell, which leaves the chunk's extremes unchanged, so one select per chunk remains
        const float4 w = a[q][u];
        const float w1 = 4 * c + 1 <= i ? w.y : w.x, w2 = 4 * c + 2 <= i ? w.z : w.x,
                    w3 = 4 * c + 3 <= i ? w.w : w.x;
        const bool cin = (c < nq) & (4 * c <= i);
        mn[q] = fminf(mn[q], cin ? fminf(fminf(w.x, w1), fminf(w2, w3)) : INFINITY);
        mx[q] = fmaxf(mx[q], cin ? fmaxf(fmaxf(w.x, w1), fmaxf(w2, w3)) : -INFINITY);
      }
    }
#pragma unroll
    for (int q = 0; q < kRowBatch; ++q) {
      mn[q] = wave_min(mn[q]);
      mx[q] = wave_max(mx[q]);
    }
    // lane q < kRowBatch: the rule of row i0 + q
    float amin = mn[0], amax = mx[0];
#pragma unroll
    for (int q = 1; q < kRowBatch; ++q)
      if (lane == q) {
        amin = mn[q];
        amax = mx[q];
      }
    int mode = kRowNone;
    float thr = 0.0f;
    if (lane < kRowBatch && i0 + lane < L) row_rule<kBoxCoxHalf>(amin, amax, eps, 0.5, tau, mode, thr);
    // keep flags and hits without per-element branches.  Cell (i0 + q, 4c + e) lies on diagonal
    // i0 - 4c + (q - e): per chunk the lane's cells fall on kDiag diagonals, counted in registers
    int32_t dc[NU][kDiag] = {};
#pragma unroll
    for (int q = 0; q < kRowBatch; ++q) {
      const int i = i0 + q;
      const int qm = __builtin_amdgcn_readlane(mode, q);  // uniform
      const float qt = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(thr), q));
      // 0/1 flags combined with bitwise operators: no branches per element.  The row's rule is
      // uniform, so the element code is written once per rule (a threshold compare, or none)
      const uint32_t all = qm == kRowAll, row_in = i < L;
      uint8_t* mrow = (true_mask && i < L && qm != kRowEach) ? true_mask + (map * L + i) * (int64_t)L : nullptr;
      auto cells = [&](auto thr_row) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int c = lane + 64 * u;
          const float v[4] = {a[q][u].x, a[q][u].y, a[q][u].z, a[q][u].w};
          uint32_t packed = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t in = row_in & (uint32_t)(c < nq) & (uint32_t)(4 * c + e <= i);
            const int32_t k1 = (int32_t)(decltype(thr_row)::value ? (in & (uint32_t)(v[e] >= qt)) : (in & all));
            dc[u][q - e + 3] += k1;
            packed |= (uint32_t)k1 << (8 * e);
          }
          vh[u] += packed;
          if (mrow && c < nq) *reinterpret_cast<uint32_t*>(mrow + 4 * c) = packed;
        }
      };
      if (qm == kRowThreshold)
        cells(std::true_type{});
      else
        cells(std::false_type{});
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int c = lane + 64 * u;
#pragma unroll
      for (int k = 0; k < kDiag; ++k) atomicAdd(&hd[dc[u][k] ? i0 - 4 * c + k - 3 : kRowMaxL + lane], dc[u][k]);
    }
    // rows with a negative or non-finite extreme: each element tested in fp64, from memory
    const uint64_t each = __ballot(lane < kRowBatch && mode == kRowEach);
    if (each) {
#pragma unroll 1
      for (int q = 0; q < kRowBatch; ++q) {
        if (!((each >> q) & 1)) continue;
        const int i = i0 + q;
        const float qmin = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(amin), q));
        const float qmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(amax), q));
        const double ymin = box_cox<kBoxCoxHalf>(qmin, eps, 0.5);
        const double range = box_cox<kBoxCoxHalf>(qmax, eps, 0.5) - ymin;
        uint8_t* mrow = true_mask ? true_mask + (map * L + i) * (int64_t)L : nullptr;
        for (int j = lane; j < L; j += 64) {
          uint8_t keep = 0;
          if (j <= i) {
            keep = (box_cox<kBoxCoxHalf>(A[(int64_t)i * L + j], eps, 0.5) - ymin) / range >= tau;
            if (keep) {
              atomicAdd(&hd[i - j], 1);
              atomicAdd(&hv[j], 1);
            }
          }
          if (mrow) mrow[j] = keep;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kRowBatch; ++q)
#pragma unroll
      for (int u = 0; u < NU; ++u) a[q][u] = an[q][u];
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int c = lane + 64 * u;
    if (c < nq)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((vh[u] >> (8 * e)) & 0xffu) atomicAdd(&hv[4 * c + e], (int32_t)((vh[u] >> (8 * e)) & 0xffu));
  }
  __syncthreads();
  for (int r = tid; r < L; r += kRowThreads) {
    const double size = (double)(L - r);
    keep_diag[map * L + r] = ((double)hd[r] / size) >= mu;
    keep_vert[map * L + r] = ((double)hv[r] / size) >= mu;
    if (diag_hits) diag_hits[map * L + r] = hd[r];
    if (vert_hits) vert_hits[map * L + r] = hv[r];
  }
}

// ---------------------------------------------------------------------------
// Averaged attention maps at the capture length ("What carries the argument":
// average attention maps of the first L positions, accumulated over the inputs;
// "Assumptions & free parameters": the batch mean stands in for each sequence):
//   maps[h][i][j] = (1/B) sum_b softmax_j(q_bhi . k_bgj * scale), j <= i; 0 above.
// One workgroup (two waves, 64 query rows) per (head, 64-row block).  Scores are
// S^T = K Q^T on MFMA (lane = query row, as in the attention kernels) over 64-key
// tiles staged in LDS.  Sequences are taken kMapChunk at a time: pass 1 finds the
// row max and 1/sum (exp2 domain) of every sequence of the chunk and keeps them in
// LDS; pass 2 walks the key tiles once, recomputes each sequence's scores and sums
// p_b / B in registers, so a map element is written once per chunk (added to the
// previous chunks' sum after the first).  No other workgroup touches these rows.
// Each pass is one software-pipelined loop over its (sequence, key tile) steps: the
// K tile and the Q fragment of step n + 1 are loaded into registers while step n is
// computed from the other LDS buffer, with one barrier per step.
// ---------------------------------------------------------------------------
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));
typedef float mf32x16 __attribute__((ext_vector_type(16)));
constexpr int kMapChunk = 16;

template <int D, bool BF16>
__global__ void __launch_bounds__(128) k_maps(const void* qv, const void* kv, int32_t B, int32_t hq, int32_t hkv,
                                              int32_t L, float scale_log2, float* maps) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  using QF = typename std::conditional<BF16, mbf16x8, float>::type;
  constexpr int QS = BF16 ? D / 16 : D / 2;           // MFMA k-steps over d
  constexpr int KSTR = BF16 ? D + 8 : D + 1;          // LDS row stride of the K tile (elements)
  constexpr int KW = 64, NKB = 2;                     // keys and 32-key blocks per key tile
  constexpr int CH = D * (int)sizeof(E) / 16;         // 16-byte chunks per key row
  constexpr int NL = KW * CH / 128;                   // chunks of a tile per thread
  __shared__ __attribute__((aligned(16))) E Ks[2][KW * KSTR];
  __shared__ float st_m[kMapChunk][128], st_il[kMapChunk][128];  // per lane: its row's max, 1/sum
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int nrb = (L + 63) / 64;
  // Workgroup k runs on XCD k % 8.  When the kv heads split evenly over the 8 XCDs, XCD x takes
  // the row blocks of kv heads x, x + 8, ... (one group at a time, heaviest row blocks first), so
  // the K tiles of a group, shared by its query heads and row blocks, stay in that XCD's L2.
  int h, rb;
  if (hkv % 8 == 0) {
    const int hpg = hq / hkv, per_group = hpg * nrb;
    const int x = (int)(blockIdx.x % 8u), slot = (int)(blockIdx.x / 8u);
    const int gl = slot / per_group, rem = slot % per_group;
    rb = nrb - 1 - rem / hpg;
    h = (x + 8 * gl) * hpg + rem % hpg;
  } else {
    h = blockIdx.x / nrb;
    rb = blockIdx.x % nrb;
  }
  const int kvh = h / (hq / hkv);
  const int i = rb * 64 + wave * 32 + r32;  // this lane's query row
  const bool row_ok = i < L;
  const float invB = 1.0f / (float)B;
  const bool vec_rows = (L & 3) == 0;  // map rows 16-byte aligned
  float* mrow = maps + ((int64_t)h * L + (row_ok ? i : 0)) * L;
  const int last = min(L, rb * 64 + 64) - 1;  // last query row (and last key) of the row block
  const int nkt = last / KW + 1;               // key tiles of this row block

  // zeros above the block diagonal (keys of the tiles past this row block)
  for (int r = 0; r < 64 && rb * 64 + r < L; ++r) {
    float* zrow = maps + ((int64_t)h * L + rb * 64 + r) * L;
    for (int jj = (rb + 1) * 64 + tid; jj < L; jj += 128) zrow[jj] = 0.0f;
  }

  auto load_q = [&](int b, QF (&qf)[QS]) {  // global -> registers
    const E* Qb = static_cast<const E*>(qv) + ((int64_t)b * hq + h) * L * (int64_t)D;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      if constexpr (BF16) {
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (row_ok) u = *reinterpret_cast<const uint4*>(Qb + (int64_t)i * D + 16 * s + 8 * g);
        qf[s] = __builtin_bit_cast(mbf16x8, u);
      } else {
        qf[s] = row_ok ? Qb[(int64_t)i * D + 2 * s + g] : 0.0f;
      }
    }
  };
  auto load_k = [&](int b, int kt, uint4 (&kr)[NL]) {  // keys kt*KW .. kt*KW+KW-1 of sequence b -> registers
    const E* Kb = static_cast<const E*>(kv) + ((int64_t)b * hkv + kvh) * L * (int64_t)D;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = tid + 128 * u, r = x / CH, c = x % CH, j = kt * KW + r;
      kr[u] = j < L ? *(reinterpret_cast<const uint4*>(Kb + (int64_t)j * D) + c) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_k = [&](int buf, const uint4 (&kr)[NL]) {  // registers -> LDS buffer
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = tid + 128 * u, r = x / CH, c = x % CH;
      E* dst = Ks[buf] + r * KSTR + c * (16 / (int)sizeof(E));
      if constexpr (BF16) {
        *reinterpret_cast<uint4*>(dst) = kr[u];
      } else {
        dst[0] = __uint_as_float(kr[u].x);
        dst[1] = __uint_as_float(kr[u].y);
        dst[2] = __uint_as_float(kr[u].z);
        dst[3] = __uint_as_float(kr[u].w);
      }
    }
  };
  // raw logits q . k of the LDS tile for this lane's row: value v of block kb is key
  // kt*KW + kb*32 + 8(v/4) + 4g + v%4.  Only the last tile of the row block holds keys past a row;
  // there they are set to -inf, which every later step keeps (the scale is positive).
  auto scores = [&](int buf, const QF (&qf)[QS], int kt, float (&x)[NKB][16]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      mf32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if constexpr (BF16) {
          const mbf16x8 kf = *reinterpret_cast<const mbf16x8*>(&Ks[buf][(kb * 32 + r32) * KSTR + 16 * s + 8 * g]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], acc, 0, 0, 0);
        } else {
          const float kf = Ks[buf][(kb * 32 + r32) * KSTR + 2 * s + g];
          acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[s], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) x[kb][v] = acc[v];
    }
    if (kt == nkt - 1) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = kt * KW + kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
          if (j > i) x[kb][v] = -INFINITY;
        }
    }
  };
  // One pass over n_steps (sequence, key tile) steps; step n is (bb, kt) = at(n).  For each step
  // `body(n, bb, kt, buf, qf)` runs on the staged tile.
  auto pipeline = [&](int n_steps, auto at, auto body) {
    QF qc[QS], qn[QS];
    uint4 kr[NL];
    int bb, kt;
    at(0, bb, kt);
    load_q(bb, qc);
    load_k(bb, kt, kr);
    store_k(0, kr);
    __syncthreads();
    for (int n = 0; n < n_steps; ++n) {
      at(n, bb, kt);
      int bn = bb, ktn = kt;
      const bool more = n + 1 < n_steps;
      if (more) {
        at(n + 1, bn, ktn);
        load_k(bn, ktn, kr);
        if (bn != bb) load_q(bn, qn);
      }
      body(n, bb, kt, n & 1, qc);
      if (more) {
        store_k((n + 1) & 1, kr);
        if (bn != bb) {
#pragma unroll
          for (int s = 0; s < QS; ++s) qc[s] = qn[s];
        }
      }
      __syncthreads();
    }
  };

  for (int b0 = 0; b0 < B; b0 += kMapChunk) {
    const int nb = min(kMapChunk, B - b0);
    // pass 1: row max and 1/sum of each sequence of the chunk (steps: sequence-major)
    float m = -INFINITY, l = 0.0f;
    pipeline(
        nb * nkt, [&](int n, int& bb, int& kt) { bb = b0 + n / nkt; kt = n % nkt; },
        [&](int n, int bb, int kt, int buf, const QF (&qf)[QS]) {
          float x[NKB][16];
          scores(buf, qf, kt, x);
          float tmax = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, x[kb][v]);
          tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));  // the row's other keys sit in lane ^ 32
          // the scaled maximum (scaling by a positive factor keeps the order); finite: key kt*KW <= i
          // for every tile of the row block
          const float mn = fmaxf(m, tmax * scale_log2);
          float part = 0.0f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) part += __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][v], scale_log2, -mn));
          part += __shfl_xor(part, 32, 64);
          l = (m == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m - mn)) + part;
          m = mn;
          if (kt == nkt - 1) {  // last tile of this sequence
            st_m[bb - b0][tid] = m;  // read back by this lane only
            st_il[bb - b0][tid] = 1.0f / l;
            m = -INFINITY;
            l = 0.0f;
          }
        });
    // pass 2: per key tile, the chunk's probabilities summed in registers (steps: tile-major)
    float acc[NKB][16];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[kb][v] = 0.0f;
    pipeline(
        nkt * nb, [&](int n, int& bb, int& kt) { kt = n / nb; bb = b0 + n % nb; },
        [&](int n, int bb, int kt, int buf, const QF (&qf)[QS]) {
          float x[NKB][16];
          scores(buf, qf, kt, x);
          const float mb = st_m[bb - b0][tid], il = st_il[bb - b0][tid];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              acc[kb][v] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][v], scale_log2, -mb)) * il;
          if (bb - b0 == nb - 1) {  // last sequence of the chunk: this key tile is complete
            if (row_ok) {
#pragma unroll
              for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                  const int j0 = kt * KW + kb * 32 + 8 * qd + 4 * g;
                  if (j0 > last) continue;  // above the block diagonal: zeros, written above
                  if (vec_rows && j0 + 3 < L) {
                    float4* dst = reinterpret_cast<float4*>(mrow + j0);
                    float4 cur = b0 == 0 ? make_float4(0.0f, 0.0f, 0.0f, 0.0f) : *dst;
                    cur.x += acc[kb][4 * qd + 0] * invB;
                    cur.y += acc[kb][4 * qd + 1] * invB;
                    cur.z += acc[kb][4 * qd + 2] * invB;
                    cur.w += acc[kb][4 * qd + 3] * invB;
                    *dst = cur;
                  } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                      if (j0 + e < L) mrow[j0 + e] = (b0 == 0 ? 0.0f : mrow[j0 + e]) + acc[kb][4 * qd + e] * invB;
                  }
                }
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[kb][v] = 0.0f;
          }
        });
  }
}

template <int D, bool BF16>
hipError_t launch_maps_t(const void* q, const void* k, int32_t B, int32_t hq, int32_t hkv, int32_t L, float scale,
                         float* maps, hipStream_t stream) {
  const int nrb = (L + 63) / 64;
  k_maps<D, BF16><<<dim3((unsigned)(hq * nrb)), dim3(128), 0, stream>>>(q, k, B, hq, hkv, L,
                                                                          scale * 1.44269504088896340736f, maps);
  return hipGetLastError();
}

// Coverage of the kept patterns inside the capture window (Referee Report major
// comments 2 and 4: agreement of the kept masks with the attention, and their
// sparsity, as the hyperparameters move): per map, the cells (i, j), j <= i < L,
// on a kept diagonal or a kept vertical, and their share of the attention mass.
// One 1024-thread workgroup per map; wave w takes rows w, w+16, ...; fp64 sums
// reduced in a fixed order (deterministic).
constexpr int kCovThreads = 1024;
__global__ void __launch_bounds__(kCovThreads)
    k_coverage(const float* maps, int32_t L, const uint8_t* keep_diag, const uint8_t* keep_vert, double* mass,
               int64_t* cells) {
  extern __shared__ uint8_t kflags[];  // [L] diagonal flags, then [L] vertical flags
  __shared__ double red_k[kCovThreads / 64], red_t[kCovThreads / 64];
  __shared__ long long red_n[kCovThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t map = blockIdx.x;
  const float* A = maps + map * (int64_t)L * L;
  for (int r = tid; r < L; r += kCovThreads) {
    kflags[r] = keep_diag[map * L + r];
    kflags[L + r] = keep_vert[map * L + r];
  }
  __syncthreads();
  double kept = 0.0, total = 0.0;
  long long n = 0;
  for (int i = wave; i < L; i += kCovThreads / 64) {
    const float* row = A + (int64_t)i * L;
    for (int jb = 0; jb <= i; jb += 4 * 64) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * 64 + lane;
        a[u] = j <= i ? row[j] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * 64 + lane;
        if (j <= i) {
          total += (double)a[u];
          if (kflags[i - j] | kflags[L + j]) {
            kept += (double)a[u];
            ++n;
          }
        }
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    kept += __shfl_xor(kept, o, 64);
    total += __shfl_xor(total, o, 64);
    n += __shfl_xor(n, o, 64);
  }
  if (lane == 0) {
    red_k[wave] = kept;
    red_t[wave] = total;
    red_n[wave] = n;
  }
  __syncthreads();
  if (tid == 0) {
    double k = 0.0, t = 0.0;
    long long c = 0;
    for (int w = 0; w < kCovThreads / 64; ++w) {
      k += red_k[w];
      t += red_t[w];
      c += red_n[w];
    }
    mass[map] = t > 0.0 ? k / t : 0.0;
    if (cells) cells[map] = c;
  }
}

// kept flags -> CSR descriptor lists at length S (entries < S).  One workgroup per
// (map, family) counts, one scans the counts over the maps, then one workgroup per
// (map, family) writes the kept indices in order: per 256-flag chunk a ballot gives
// each kept flag its rank among the kept flags before it.
constexpr int kDescThreads = 256;
__global__ void __launch_bounds__(kDescThreads)
    k_desc_count(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t L, int32_t S, int32_t* diag_ptr,
                 int32_t* vert_ptr) {
  __shared__ int32_t red[kDescThreads / 64];
  const int m = blockIdx.x >> 1, fam = blockIdx.x & 1;
  const uint8_t* f = (fam == 0 ? keep_diag : keep_vert) + (int64_t)m * L;
  const int32_t Lc = min(L, S);
  int32_t c = 0;
  for (int x = threadIdx.x; x < Lc; x += kDescThreads) c += f[x] != 0;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int w = 0; w < kDescThreads / 64; ++w) t += red[w];
    (fam == 0 ? diag_ptr : vert_ptr)[m + 1] = t;
  }
}

__global__ void k_desc_scan(int32_t n_maps, int32_t* diag_ptr, int32_t* vert_ptr) {
  int32_t* p = threadIdx.x == 0 ? diag_ptr : vert_ptr;
  p[0] = 0;
  for (int m = 0; m < n_maps; ++m) p[m + 1] += p[m];
}

__global__ void __launch_bounds__(kDescThreads)
    k_desc_fill(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t L, int32_t S, const int32_t* diag_ptr,
                int32_t* diag_off, const int32_t* vert_ptr, int32_t* vert_col) {
  __shared__ int32_t wcount[kDescThreads / 64];
  const int m = blockIdx.x >> 1, fam = blockIdx.x & 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* f = (fam == 0 ? keep_diag : keep_vert) + (int64_t)m * L;
  int32_t* out = fam == 0 ? diag_off : vert_col;
  int32_t base = (fam == 0 ? diag_ptr : vert_ptr)[m];
  const int32_t Lc = min(L, S);
  for (int32_t c0 = 0; c0 < Lc; c0 += kDescThreads) {
    const int32_t x = c0 + tid;
    const bool on = x < Lc && f[x] != 0;
    const unsigned long long bal = __ballot(on);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int32_t before = 0, total = 0;
    for (int w = 0; w < kDescThreads / 64; ++w) {
      before += w < wave ? wcount[w] : 0;
      total += wcount[w];
    }
    if (on) out[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = x;
    base += total;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_capture(const float* maps, int32_t n_maps, int32_t L, double lambda, double eps, double tau,
                          double mu, int32_t norm_scope, uint8_t* keep_diag, uint8_t* keep_vert, int32_t* diag_hits,
                          int32_t* vert_hits, uint8_t* true_mask, hipStream_t stream) {
  if (lambda == 0.5 && norm_scope == 0 && L <= kRowMaxL && L % 4 == 0) {
    hipLaunchKernelGGL(k_capture_rows, dim3((unsigned)n_maps), dim3(kRowThreads), 0, stream, maps, L, eps, tau, mu,
                       keep_diag, keep_vert, diag_hits, vert_hits, true_mask);
    return hipGetLastError();
  }
  const size_t lds = 6 * sizeof(int32_t) * (size_t)L;  // hits, then per-row min, max, threshold, mode
  auto kern = lambda == 0.5 ? k_capture<kBoxCoxHalf> : lambda == 0.0 ? k_capture<kBoxCoxLog> : k_capture<kBoxCoxPow>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)n_maps), dim3(kThreads), lds, stream, maps, L, lambda, eps, tau, mu,
                     norm_scope, keep_diag, keep_vert, diag_hits, vert_hits, true_mask);
  return hipGetLastError();
}

hipError_t launch_attention_maps(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t L,
                                 int32_t head_dim, int32_t dtype, float scale, float* maps, hipStream_t stream) {
  if (dtype == SA_DTYPE_BF16)
    return head_dim == 64 ? launch_maps_t<64, true>(q, k, batch, hq, hkv, L, scale, maps, stream)
                          : launch_maps_t<128, true>(q, k, batch, hq, hkv, L, scale, maps, stream);
  return head_dim == 64 ? launch_maps_t<64, false>(q, k, batch, hq, hkv, L, scale, maps, stream)
                        : launch_maps_t<128, false>(q, k, batch, hq, hkv, L, scale, maps, stream);
}

hipError_t launch_coverage(const float* maps, int32_t n_maps, int32_t L, const uint8_t* keep_diag,
                           const uint8_t* keep_vert, double* mass, int64_t* cells, hipStream_t stream) {
  hipLaunchKernelGGL(k_coverage, dim3((unsigned)n_maps), dim3(kCovThreads), 2 * (size_t)L, stream, maps, L, keep_diag,
                     keep_vert, mass, cells);
  return hipGetLastError();
}

hipError_t launch_patterns_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L,
                                   int32_t S, int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr,
                                   int32_t* vert_col, hipStream_t stream) {
  hipLaunchKernelGGL(k_desc_count, dim3((unsigned)(2 * n_maps)), dim3(kDescThreads), 0, stream, keep_diag, keep_vert, L,
                     S, diag_ptr, vert_ptr);
  hipLaunchKernelGGL(k_desc_scan, dim3(1), dim3(2), 0, stream, n_maps, diag_ptr, vert_ptr);
  hipLaunchKernelGGL(k_desc_fill, dim3((unsigned)(2 * n_maps)), dim3(kDescThreads), 0, stream, keep_diag, keep_vert, L,
                     S, diag_ptr, diag_off, vert_ptr, vert_col);
  return hipGetLastError();
}

}  // namespace sa
