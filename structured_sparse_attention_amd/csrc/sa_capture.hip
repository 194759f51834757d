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
// Layout: at lambda = 0.5 with per-row extremes and L <= 512 (the pages' case), k_capture_tiles reads
// the causal half once, through LDS tiles of 16 rows (described above it).  Every other case runs
// k_capture: one 1024-thread workgroup per map.  Pass 1: the fp32 min/max of every row (wave w takes
// rows w, w+16, ..., four rows at a time, lanes over columns); pass 2: one thread per row transforms
// the extremes and finds the threshold; pass 3: the element pass (lanes over columns, four loads in
// flight per lane), hits accumulating with LDS atomics.  That kernel reads the causal half twice.
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
  // the row maximum's score is (ymax - ymin) / range = range / range = 1 exactly (same fp64 steps)
  if (!(1.0 >= tau)) {
    mode = kRowNone;
    return;
  }
  mode = kRowThreshold;
  uint32_t lo = bmin, hi = bmax;  // the answer lies in [lo, hi], and hi passes
  if constexpr (KIND == kBoxCoxHalf) {
    const double sr = 1.0 + 0.5 * (ymin + tau * range);
    const double a = sr > 0.0 ? sr * sr - eps : 0.0;
    const uint32_t c = a <= (double)amin ? bmin : a >= (double)amax ? bmax : __float_as_uint((float)a);
    // c and its two neighbours tested together (three independent evaluations instead of a chain);
    // a passing value bounds the answer from above, a failing one from below
    const uint32_t cm = c > lo ? c - 1 : c, cp = c < hi ? c + 1 : c;
    const bool qm = pass(cm), qc = pass(c), qp = pass(cp);
    if (qp) hi = cp;
    else lo = cp + 1;
    if (qc) hi = c;
    else lo = max(lo, c + 1);
    if (qm) hi = cm;
    else lo = max(lo, cm + 1);
    if (qc) {
      for (int k = 0; k < 8 && hi > lo; ++k) {
        if (!pass(hi - 1)) {
          lo = hi;  // hi passes and the float below it does not
          break;
        }
        --hi;
      }
    } else {
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

constexpr int kRowMaxL = 512;  // longest map the tiled single-read kernel takes

// ---------------------------------------------------------------------------
// Tiled single read of the map (k_capture_tiles): the same keep flags and hits as k_capture for
// lambda = 0.5, per-row extremes and L <= 512 with L % 4 == 0.  512 threads per map take the causal
// half in chunks of 16 rows, in a pipeline (two maps share a CU, so each covers the other's waits):
//   chunk n      is counted from LDS tile n % 2 with its rules;
//   chunk n + 1  waits in the other tile with its extremes, and one wave finds its 16 row rules
//                (lane = row, row_rule) while the others count chunk n;
//   chunks n + 2 and n + 3  are in flight into two register sets: thread (row t = tid / 32, phase
//                s = tid % 32) loads float4 columns s + 32k of chunk row t; when chunk n + 2 lands,
//                the registers go to the tile chunk n has freed and its extremes come from the same
//                values (32-lane reductions; min and max are exact in any order), and the loads of
//                chunk n + 4 take their place (two chunks of time to arrive).
// Hits: lane `col` counts column col (vertical hits) and diagonal offset col (cell (i, i - col) of
// chunk row t sits at tile[t][i - col]): each counter belongs to one lane for the whole map and stays
// in a register, so no atomics.  A wave whose columns all lie past a chunk's last row skips it; the
// rule wave is the last wave, which has no cells in most chunks.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 16, kTileThreads = 512;

__global__ void __launch_bounds__(kTileThreads)
    k_capture_tiles(const float* maps, int32_t L, double eps, double tau, double mu, uint8_t* keep_diag,
                    uint8_t* keep_vert, int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask) {
#pragma clang fp contract(off)
  constexpr int PH = kTileThreads / kTileRows;  // threads per chunk row: 32
  constexpr int NK = kRowMaxL / (4 * PH);       // float4 per thread and chunk: 4
  constexpr int kRuleWave = kTileThreads / 64 - 1;
  static_assert(kTileThreads == kRowMaxL && PH * NK * 4 == kRowMaxL, "lane = column = diagonal offset");
  // tile[b][0] is a guard row: a diagonal lane reads row t at column i0 + t - r, which lies in row t - 1
  // (or the guard row) when r > i0 + t.  Non-causal cells (column > row, past L) and the guard rows
  // hold NaN, which fails every threshold compare, so the whole-chunk hit pass needs no range tests.
  __shared__ __attribute__((aligned(16))) float tile[2][kTileRows + 1][kRowMaxL];
  __shared__ float ex_min[2][kTileRows], ex_max[2][kTileRows];
  __shared__ int32_t rl_mode[2][kTileRows], rl_fast[2];
  __shared__ __attribute__((aligned(16))) float rl_thr[2][kTileRows];
  __shared__ double rl_ymin[2][kTileRows], rl_range[2][kTileRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t_ld = tid / PH, s_ld = tid % PH;
  const int64_t map = blockIdx.x;
  const float* A = maps + map * (int64_t)L * L;
  const int nq = L / 4;  // float4 per row
  const uint32_t map_bytes = (uint32_t)L * L * 4u;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, map_bytes, 0x00020000);
  const int nch = (L + kTileRows - 1) / kTileRows;
  // causal cells of chunk row t; cells past the row's last float4, the map or the rows read as zero
  float4 ra[NK], rb[NK];
  auto load_chunk = [&](int n, float4(&a)[NK]) {
    const int i = n * kTileRows + t_ld;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = s_ld + PH * k;
      const uint32_t off = (i < L && c < nq && 4 * c <= i) ? (uint32_t)(i * L + 4 * c) * 4u : map_bytes;
      a[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rsA, off, 0, 0));
    }
  };
  // chunk row t_ld from the registers into tile `buf`, its non-causal cells (column > row, past L) as
  // NaN, and its extremes from the same values: fminf and fmaxf skip NaN, so the masked cells leave
  // them unchanged (as do NaN cells of the map itself)
  auto land_chunk = [&](int n, int buf, const float4(&a)[NK]) {
    const int i = n * kTileRows + t_ld;
    const float nan = __builtin_nanf("");
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = s_ld + PH * k;
      const bool cv = (i < L) & (c < nq);
      const float4 w = a[k];
      const float4 st = make_float4(cv & (4 * c <= i) ? w.x : nan, cv & (4 * c + 1 <= i) ? w.y : nan,
                                    cv & (4 * c + 2 <= i) ? w.z : nan, cv & (4 * c + 3 <= i) ? w.w : nan);
      mn = fminf(mn, fminf(fminf(st.x, st.y), fminf(st.z, st.w)));
      mx = fmaxf(mx, fmaxf(fmaxf(st.x, st.y), fmaxf(st.z, st.w)));
      *reinterpret_cast<float4*>(&tile[buf][t_ld + 1][4 * c]) = st;
    }
#pragma unroll
    for (int o = PH / 2; o > 0; o >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, o, PH));
      mx = fmaxf(mx, __shfl_xor(mx, o, PH));
    }
    if (s_ld == 0) {
      ex_min[n & 1][t_ld] = mn;
      ex_max[n & 1][t_ld] = mx;
    }
  };
  // the rule wave: row rules of chunk n (lane = row)
  auto rules = [&](int n) {
    if (wave != kRuleWave || lane >= kTileRows) return;
    // the rule chain (dependent fp64 steps) paces the pipeline: issue it ahead of the counting waves
    // that share its SIMD
    __builtin_amdgcn_s_setprio(3);
    int mode = kRowNone;
    float thr = 0.0f;
    double ymin = 0.0, range = 0.0;
    if (n * kTileRows + lane < L) {
      const float amin = ex_min[n & 1][lane], amax = ex_max[n & 1][lane];
      row_rule<kBoxCoxHalf>(amin, amax, eps, 0.5, tau, mode, thr);
      if (mode == kRowEach) {
        ymin = box_cox<kBoxCoxHalf>(amin, eps, 0.5);
        range = box_cox<kBoxCoxHalf>(amax, eps, 0.5) - ymin;
      }
    }
    rl_mode[n & 1][lane] = mode;
    rl_thr[n & 1][lane] = thr;
    rl_ymin[n & 1][lane] = ymin;
    rl_range[n & 1][lane] = range;
    // every row of the chunk decided by its threshold (rows past L are never visited)
    const uint64_t thr_rows = __ballot(mode == kRowThreshold || n * kTileRows + lane >= L);
    if (lane == 0) rl_fast[n & 1] = (thr_rows & ((1ull << kTileRows) - 1)) == ((1ull << kTileRows) - 1);
    __builtin_amdgcn_s_setprio(0);
  };
  const int col = 64 * wave + lane;  // this lane's column and diagonal offset
  int32_t hv = 0, hd = 0;

  // prologue: guard rows; chunk 0 landed and ruled, chunk 1 landed, chunks 2 and 3 in flight (ra holds
  // the even chunks, rb the odd ones)
  tile[0][0][tid] = __builtin_nanf("");
  tile[1][0][tid] = __builtin_nanf("");
  load_chunk(0, ra);
  if (nch > 1) load_chunk(1, rb);
  land_chunk(0, 0, ra);
  if (nch > 2) load_chunk(2, ra);
  __syncthreads();
  rules(0);
  if (nch > 1) {
    land_chunk(1, 1, rb);
    if (nch > 3) load_chunk(3, rb);
  }
  __syncthreads();
  auto step = [&](int n, float4(&a)[NK]) {  // a: the registers of chunk n + 2 (same parity as n)
    if (n + 1 < nch) rules(n + 1);
    // ---- hits of chunk n
    const int i0 = n * kTileRows, rows = min(kTileRows, L - i0);
    const float* tl = &tile[n & 1][1][0];  // chunk row 0
    const float thr_v = rl_thr[n & 1][lane % kTileRows];
    if (true_mask == nullptr && rl_fast[n & 1] && rows == kTileRows) {
      // a whole chunk, every row by its threshold: the lane's cells of a few rows are read first, then
      // each counts iff it is at or above its row's threshold (cells outside the causal rows are NaN)
      if (64 * wave <= i0 + kTileRows - 1) {
        const float* bv = tl + col;         // column col of row t: bv[t * kRowMaxL]
        const float* bd = tl + (i0 - col);  // diagonal col of row t: bd[t * (kRowMaxL + 1)]
        const float4* th = reinterpret_cast<const float4*>(&rl_thr[n & 1][0]);  // same address in every lane
#pragma unroll
        for (int g = 0; g < kTileRows / 4; ++g) {
          float v[4], w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            v[t] = bv[(4 * g + t) * kRowMaxL];
            w[t] = bd[(4 * g + t) * (kRowMaxL + 1)];
          }
          const float4 t4 = th[g];
          hv += (int32_t)(v[0] >= t4.x) + (int32_t)(v[1] >= t4.y) + (int32_t)(v[2] >= t4.z) + (int32_t)(v[3] >= t4.w);
          hd += (int32_t)(w[0] >= t4.x) + (int32_t)(w[1] >= t4.y) + (int32_t)(w[2] >= t4.z) + (int32_t)(w[3] >= t4.w);
        }
      }
    } else if (!(64 * wave > i0 + rows - 1 && true_mask == nullptr)) {
      const int mode_v = rl_mode[n & 1][lane % kTileRows];
      for (int t = 0; t < rows; ++t) {
        const int i = i0 + t;
        const int m = __builtin_amdgcn_readlane(mode_v, t);
        const float thr = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(thr_v), t));
        // column col <= i, and offset col <= i (its column i - col >= 0)
        const bool in = col <= i;
        const float v = tl[t * kRowMaxL + col];
        const float w = tl[t * kRowMaxL + max(i - col, 0)];
        int32_t kv = 0, kd = 0;
        if (m == kRowThreshold) {
          kv = in & (v >= thr);
          kd = in & (w >= thr);
        } else if (m == kRowAll) {
          kv = in;
          kd = in;
        } else if (m == kRowEach) {
          const double ymin = rl_ymin[n & 1][t], range = rl_range[n & 1][t];
          kv = in && (box_cox<kBoxCoxHalf>(v, eps, 0.5) - ymin) / range >= tau;
          kd = in && (box_cox<kBoxCoxHalf>(w, eps, 0.5) - ymin) / range >= tau;
        }
        hv += kv;
        hd += kd;
        if (true_mask != nullptr && col < L) true_mask[(map * L + i) * (int64_t)L + col] = (uint8_t)kv;
      }
    }
    __syncthreads();  // chunk n counted: its tile is free; rules of chunk n + 1 written
    if (n + 2 < nch) {
      land_chunk(n + 2, n & 1, a);
      if (n + 4 < nch) load_chunk(n + 4, a);
    }
    __syncthreads();  // chunk n + 2 in its tile
  };
  for (int n = 0; n < nch; n += 2) {
    step(n, ra);
    if (n + 1 < nch) step(n + 1, rb);
  }
  if (col < L) {
    const double size = (double)(L - col);
    keep_diag[map * L + col] = ((double)hd / size) >= mu;
    keep_vert[map * L + col] = ((double)hv / size) >= mu;
    if (diag_hits) diag_hits[map * L + col] = hd;
    if (vert_hits) vert_hits[map * L + col] = hv;
  }
}

// ---------------------------------------------------------------------------
// Averaged attention maps at the capture length ("What carries the argument":
// average attention maps of the first L positions, accumulated over the inputs;
// "Assumptions & free parameters": the batch mean stands in for each sequence):
//   maps[h][i][j] = (1/B) sum_b softmax_j(q_bhi . k_bgj * scale), j <= i; 0 above.
// One workgroup (four waves) per (head, pair of 64-row blocks): waves 0-1 take the
// lower block, waves 2-3 the upper one, and both share every K tile (the lower block's
// waves skip the upper block's diagonal tile).  Scores are S^T = K Q^T on MFMA (lane =
// query row, as in the attention kernels) over 64-key tiles staged in LDS.  Sequences
// are taken kMapChunk at a time: pass 1 finds the row max and sum (exp2 domain) of
// every sequence of the chunk and keeps max + log2 sum in LDS; pass 2 walks the key
// tiles once, recomputes each sequence's scores and sums p_b / B in registers, so a
// map element is written once per chunk (added to the previous chunks' sum after the
// first).  No other workgroup touches these rows.
// Each pass is one software-pipelined loop over its (sequence, key tile) steps: the
// K tile and the Q fragment of step n + 1 are loaded into registers while step n is
// computed from the other LDS buffer, with one barrier per step.
// ---------------------------------------------------------------------------
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));
typedef float mf32x16 __attribute__((ext_vector_type(16)));
constexpr int kMapChunk = 16;
constexpr int kMapThreads = 256;  // four waves: two row blocks of 64 query rows

template <int D, bool BF16>
__global__ void __launch_bounds__(kMapThreads) __attribute__((amdgpu_waves_per_eu(3)))
k_maps(const void* qv, const void* kv, int32_t B, int32_t hq, int32_t hkv, int32_t L, float scale_log2, float* maps) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  using QF = typename std::conditional<BF16, mbf16x8, float>::type;
  constexpr int QS = BF16 ? D / 16 : D / 2;           // MFMA k-steps over d
  constexpr int KSTR = BF16 ? D + 8 : D + 1;          // LDS row stride of the K tile (elements)
  constexpr int KW = 64, NKB = 2;                     // keys and 32-key blocks per key tile
  constexpr int CH = D * (int)sizeof(E) / 16;         // 16-byte chunks per key row
  constexpr int NL = KW * CH / kMapThreads;           // chunks of a tile per thread
  __shared__ __attribute__((aligned(16))) E Ks[2][KW * KSTR];
  // per lane: its row's max less log2 of its sum, per sequence of the chunk, so that pass 2's
  // probability is one exp2 (p = 2^(x scale - max) / sum = 2^(x scale - (max + log2 sum)))
  __shared__ float st_m[kMapChunk][kMapThreads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int nrb = (L + 63) / 64;
  const int npr = (nrb + 1) / 2;  // pairs of row blocks, one per workgroup
  // Workgroup k runs on XCD k % 8.  When the kv heads split evenly over the 8 XCDs, XCD x takes
  // the row blocks of kv heads x, x + 8, ... (one group at a time, heaviest row blocks first), so
  // the K tiles of a group, shared by its query heads and row blocks, stay in that XCD's L2.
  int h, pr;
  if (hkv % 8 == 0) {
    const int hpg = hq / hkv, per_group = hpg * npr;
    const int x = (int)(blockIdx.x % 8u), slot = (int)(blockIdx.x / 8u);
    const int gl = slot / per_group, rem = slot % per_group;
    pr = npr - 1 - rem / hpg;
    h = (x + 8 * gl) * hpg + rem % hpg;
  } else {
    h = blockIdx.x / npr;
    pr = blockIdx.x % npr;
  }
  const int kvh = h / (hq / hkv);
  // waves 0-1 take row block 2 pr, waves 2-3 row block 2 pr + 1 (absent past the map): both share the
  // workgroup's K tiles
  const int rb = 2 * pr + (wave >> 1);
  const int i = rb * 64 + (wave & 1) * 32 + r32;  // this lane's query row
  const bool row_ok = rb < nrb && i < L;
  const float invB = 1.0f / (float)B;
  const bool vec_rows = (L & 3) == 0;  // map rows 16-byte aligned
  float* mrow = maps + ((int64_t)h * L + (row_ok ? i : 0)) * L;
  const int last = min(L, rb * 64 + 64) - 1;          // last query row (and last key) of this wave's row block
  const int nkt_w = rb < nrb ? last / KW + 1 : 0;     // key tiles of this wave's row block
  const int nkt = (min(L, 2 * pr * 64 + 128) - 1) / KW + 1;  // key tiles of the workgroup (its upper block)

  // zeros above the block diagonal (keys of the tiles past each row block)
  for (int q = 0; q < 2; ++q) {
    const int rq = 2 * pr + q;
    for (int r = 0; r < 64 && rq * 64 + r < L; ++r) {
      float* zrow = maps + ((int64_t)h * L + rq * 64 + r) * L;
      for (int jj = (rq + 1) * 64 + tid; jj < L; jj += kMapThreads) zrow[jj] = 0.0f;
    }
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
      const int x = tid + kMapThreads * u, r = x / CH, c = x % CH, j = kt * KW + r;
      kr[u] = j < L ? *(reinterpret_cast<const uint4*>(Kb + (int64_t)j * D) + c) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_k = [&](int buf, const uint4 (&kr)[NL]) {  // registers -> LDS buffer
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = tid + kMapThreads * u, r = x / CH, c = x % CH;
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
    if (kt == nkt_w - 1) {
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
          if (kt >= nkt_w) return;  // the upper block's diagonal tile lies above this wave's rows
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
          if (kt == nkt_w - 1) {  // last tile of this sequence for this wave's rows
            st_m[bb - b0][tid] = m + __builtin_amdgcn_logf(l);  // read back by this lane only
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
          if (kt >= nkt_w) return;  // nothing of this wave's rows in the tile (acc stays zero)
          float x[NKB][16];
          scores(buf, qf, kt, x);
          const float mb = st_m[bb - b0][tid];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[kb][v] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][v], scale_log2, -mb));
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
  const int npr = (nrb + 1) / 2;
  k_maps<D, BF16><<<dim3((unsigned)(hq * npr)), dim3(kMapThreads), 0, stream>>>(q, k, B, hq, hkv, L,
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
    hipLaunchKernelGGL(k_capture_tiles, dim3((unsigned)n_maps), dim3(kTileThreads), 0, stream, maps, L, eps, tau, mu,
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
