// sa_sample.hip -- runtime capture from sampled query rows, and pattern selection, on gfx950.
//
// "SampleAttention: Near-Lossless Acceleration of Long Context LLM Inference with
// Adaptive Structured Sparse Attention", abstract: head-specific sparse patterns
// are captured at runtime, per input, at low cost.  Here a contiguous block of the
// input's own query rows takes its causal softmax over all keys, and each row's
// probabilities are added onto the pattern pool of the Pith review of "DAM:
// Dynamic Attention Mask for Long-Context Large Language Model Inference
// Acceleration" ("What carries the argument": diagonals j = i - r, verticals j = c):
//   diag[h][r] += p_i(i - r),   vert[h][c] += p_i(c),
// over the pairs not covered yet: outside the local window (i - j >= band) and off
// the columns already kept.  The selection keeps, for one family, the fewest
// top-scoring patterns that bring the covered mass of the sampled rows to a
// fraction alpha (ties at the threshold all kept); it runs for the columns first,
// then for the diagonals rescored on the mass the columns leave.
//
// Scores are fixed point (int64, unit 2^-32) so that every sum is an integer sum:
// the totals do not depend on the order of the atomics, and the selection is
// exact integer arithmetic.
//
// k_sample_lse: one workgroup of 8 waves per (sequence, head, 32 sampled rows);
//   lane = query row, 32-key tiles split over the waves, S^T = K Q^T on MFMA,
//   online max/sum per lane, merged across waves in LDS.
// k_sample_acc: one workgroup of 4 waves per (head, 64-key tile); the tile is staged
//   in LDS per sequence, the waves take 32-row chunks, recompute the scores and add
//   p = exp2(s - lse) into LDS: diagonals with int64 LDS atomics (a row chunk and a
//   key tile touch n_rows + 63 diagonals), verticals in registers; then one global
//   int64 atomic per touched pattern.
// k_select: one 1024-thread workgroup per head; the threshold is found by
//   a most-significant-digit radix search over the score bits (8-bit digits), each
//   pass a mass histogram of the scores inside the current bucket.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 sbf16x8 __attribute__((ext_vector_type(8)));
typedef float sf32x16 __attribute__((ext_vector_type(16)));
constexpr double kFixUnit = 4294967296.0;  // 2^32 per unit of probability mass
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

template <bool BF16>
struct SampleTypes {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  using QF = typename std::conditional<BF16, sbf16x8, float>::type;
};

// B-operand fragments of query row i (zero when the row is outside the sample)
template <int D, bool BF16>
__device__ inline void load_q_frags(const typename SampleTypes<BF16>::E* Qrow, bool ok, int g,
                                    typename SampleTypes<BF16>::QF (&qf)[BF16 ? D / 16 : D / 2]) {
  constexpr int QS = BF16 ? D / 16 : D / 2;
#pragma unroll
  for (int s = 0; s < QS; ++s) {
    if constexpr (BF16) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (ok) u = *reinterpret_cast<const uint4*>(Qrow + 16 * s + 8 * g);
      qf[s] = __builtin_bit_cast(sbf16x8, u);
    } else {
      qf[s] = ok ? Qrow[2 * s + g] : 0.0f;
    }
  }
}

template <int D, bool BF16>
__global__ void __launch_bounds__(512) k_sample_lse(const void* qv, const void* kv, int32_t hq, int32_t hkv, int32_t S,
                                                    int32_t row0, int32_t n_rows, float scale_log2, float* row_lse) {
  using E = typename SampleTypes<BF16>::E;
  using QF = typename SampleTypes<BF16>::QF;
  constexpr int QS = BF16 ? D / 16 : D / 2;
  __shared__ float red_m[8][32], red_l[8][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int nch = (n_rows + 31) / 32;
  const int ch = blockIdx.x % nch;
  const int h = (blockIdx.x / nch) % hq;
  const int b = blockIdx.x / (nch * hq);
  const int kvh = h / (hq / hkv);
  const int n = ch * 32 + r32;  // this lane's sampled row, as an index into the sample
  const bool row_ok = n < n_rows;
  const int i = row0 + (row_ok ? n : 0);
  const int i_last = row0 + min(ch * 32 + 31, n_rows - 1);
  const E* Q = static_cast<const E*>(qv) + (((int64_t)b * hq + h) * S + i) * (int64_t)D;
  const E* K = static_cast<const E*>(kv) + ((int64_t)b * hkv + kvh) * (int64_t)S * D;
  QF qf[QS];
  load_q_frags<D, BF16>(Q, row_ok, g, qf);

  float m = -INFINITY, l = 0.0f;
  for (int kt = wave; kt * 32 <= i_last; kt += 8) {
    const int key = kt * 32 + r32;  // A-operand row supplied by this lane
    const E* Krow = K + (int64_t)min(key, S - 1) * D;
    sf32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      if constexpr (BF16) {
        const sbf16x8 kf = __builtin_bit_cast(sbf16x8, *reinterpret_cast<const uint4*>(Krow + 16 * s + 8 * g));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Krow[2 * s + g], qf[s], acc, 0, 0, 0);
      }
    }
    float x[16], tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = kt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      x[v] = (row_ok && j <= i) ? acc[v] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));  // the row's other keys of the tile sit in lane ^ 32
    const float mn = fmaxf(m, tmax);
    if (mn == -INFINITY) continue;  // nothing of this row seen yet
    float part = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) part += __builtin_amdgcn_exp2f(x[v] - mn);
    part += __shfl_xor(part, 32, 64);
    l = (m == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m - mn)) + part;
    m = mn;
  }
  if (g == 0) {
    red_m[wave][r32] = m;
    red_l[wave][r32] = l;
  }
  __syncthreads();
  if (wave == 0 && g == 0 && row_ok) {
    float M = -INFINITY;
    for (int w = 0; w < 8; ++w) M = fmaxf(M, red_m[w][r32]);
    float L = 0.0f;
    for (int w = 0; w < 8; ++w)
      if (red_m[w][r32] != -INFINITY) L += red_l[w][r32] * __builtin_amdgcn_exp2f(red_m[w][r32] - M);
    row_lse[((int64_t)b * hq + h) * n_rows + n] = (M + __log2f(L)) * kLn2;
  }
}

template <int D, bool BF16>
__global__ void __launch_bounds__(256) k_sample_acc(const void* qv, const void* kv, int32_t B, int32_t hq, int32_t hkv,
                                                    int32_t S, int32_t row0, int32_t n_rows, int32_t band,
                                                    const uint8_t* skip_cols, float scale_log2, const float* row_lse,
                                                    unsigned long long* diag_score, unsigned long long* vert_score) {
  using E = typename SampleTypes<BF16>::E;
  using QF = typename SampleTypes<BF16>::QF;
  constexpr int QS = BF16 ? D / 16 : D / 2;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;  // LDS row stride of the key tile (elements)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* Ks = reinterpret_cast<E*>(smem);
  unsigned long long* vacc_lds = reinterpret_cast<unsigned long long*>(smem + 64 * KSTR * sizeof(E));
  unsigned long long* dacc = vacc_lds + 64;  // [n_rows + 63] diagonals r = r_base + x
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int ntile = (row0 + n_rows - 1) / 64 + 1;
  const int h = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int kvh = h / (hq / hkv);
  const int c0 = tile * 64;
  const int r_base = row0 - c0 - 63;
  const int span = n_rows + 63;
  const int nch = (n_rows + 31) / 32;
  // rows i < c0 + band see no key of this tile outside their window
  if (row0 + n_rows - 1 < c0 + band) return;
  for (int x = tid; x < span; x += 256) dacc[x] = 0ull;
  if (tid < 64) vacc_lds[tid] = 0ull;
  float vacc[2][16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) vacc[kb][v] = 0.0f;
  // columns of this tile already kept (their pairs are covered); staged once
  __shared__ uint8_t skip_lds[64];
  const uint8_t* skip = nullptr;
  if (skip_cols) {
    if (tid < 64) skip_lds[tid] = (c0 + tid < S) ? skip_cols[(int64_t)h * S + c0 + tid] : 1;
    skip = skip_lds;
  }

  for (int b = 0; b < B; ++b) {
    const E* K = static_cast<const E*>(kv) + ((int64_t)b * hkv + kvh) * (int64_t)S * D;
    __syncthreads();
    constexpr int CH = D * (int)sizeof(E) / 16;  // 16-byte chunks per key row
    for (int x = tid; x < 64 * CH; x += 256) {
      const int r = x / CH, c = x % CH, j = c0 + r;
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (j < S) u = *(reinterpret_cast<const uint4*>(K + (int64_t)j * D) + c);
      E* dst = Ks + r * KSTR + c * (16 / (int)sizeof(E));
      if constexpr (BF16) {
        *reinterpret_cast<uint4*>(dst) = u;
      } else {
        dst[0] = __uint_as_float(u.x);
        dst[1] = __uint_as_float(u.y);
        dst[2] = __uint_as_float(u.z);
        dst[3] = __uint_as_float(u.w);
      }
    }
    __syncthreads();
    for (int ch = wave; ch < nch; ch += 4) {
      const int n = ch * 32 + r32;
      const bool row_ok = n < n_rows;
      const int i = row0 + (row_ok ? n : 0);
      if (row0 + ch * 32 + 31 < c0 + band) continue;  // no row of the chunk reaches the tile outside its window
      QF qf[QS];
      load_q_frags<D, BF16>(static_cast<const E*>(qv) + (((int64_t)b * hq + h) * S + i) * (int64_t)D, row_ok, g, qf);
      const float lse2 = row_ok ? row_lse[((int64_t)b * hq + h) * n_rows + n] * kLog2e : 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sf32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          if constexpr (BF16) {
            const sbf16x8 kf = *reinterpret_cast<const sbf16x8*>(&Ks[(kb * 32 + r32) * KSTR + 16 * s + 8 * g]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], acc, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[(kb * 32 + r32) * KSTR + 2 * s + g], qf[s], acc, 0, 0, 0);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = c0 + kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
          if (row_ok && j <= i - band && !(skip && skip[j - c0])) {
            const float p = __builtin_amdgcn_exp2f(acc[v] * scale_log2 - lse2);
            vacc[kb][v] += p;
            const unsigned long long fx = (unsigned long long)__double2ll_rn((double)p * kFixUnit);
            if (fx) atomicAdd(&dacc[i - j - r_base], fx);
          }
        }
      }
    }
  }
  // verticals: each lane's partial sum over its rows, in fixed point, summed over the lanes
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const unsigned long long fx = (unsigned long long)__double2ll_rn((double)vacc[kb][v] * kFixUnit);
      if (fx) atomicAdd(&vacc_lds[kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3)], fx);
    }
  __syncthreads();
  unsigned long long* dg = diag_score + (int64_t)h * S;
  unsigned long long* vt = vert_score + (int64_t)h * S;
  for (int x = tid; x < span; x += 256) {
    const int r = r_base + x;
    if (dacc[x] && r >= 0 && r < S) atomicAdd(&dg[r], dacc[x]);
  }
  if (tid < 64 && c0 + tid < S && vacc_lds[tid]) atomicAdd(&vt[c0 + tid], vacc_lds[tid]);
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;

__device__ inline long long block_sum_ll(long long x, long long* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) t += red[w];
  return t;
}

__device__ inline long long block_max_ll(long long x, long long* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) t = max(t, red[w]);
  return t;
}

__global__ void __launch_bounds__(kSelThreads)
    k_select(const long long* scores, int32_t S, double alpha, long long t_all, int32_t band, uint8_t* keep_out) {
  __shared__ long long red[kSelThreads / 64];
  __shared__ unsigned long long hist[256];
  __shared__ long long sh_state[2];  // chosen digit, new mass above
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const long long* v = scores + (int64_t)h * S;
  uint8_t* keep = keep_out + (int64_t)h * S;

  long long tot = 0, mx = 0;
  for (int x = tid; x < S; x += kSelThreads) {
    const long long a = v[x];
    tot += a;
    mx = max(mx, a);
  }
  tot = block_sum_ll(tot, red);
  mx = block_max_ll(mx, red);
  // mass still to cover: the scores hold what is not covered yet
  const long long need = (long long)ceil(alpha * (double)t_all) - (t_all - tot);
  long long theta = 0x7fffffffffffffffLL;  // need <= 0: nothing more is kept
  if (need > tot) {
    theta = 1;  // every pattern falls short together: all with mass are kept
  } else if (need > 0) {
    long long prefix = 0, above = 0;
    int hi = 64 - __clzll((unsigned long long)mx);  // bit length of the largest score
    while (hi > 0) {
      const int lo = max(hi - 8, 0), width = hi - lo;
      const unsigned long long nbins = 1ull << width;
      if (tid < 256) hist[tid] = 0ull;
      __syncthreads();
      long long zero_bin = 0;  // the most populated bin is summed in registers
      for (int x = tid; x < S; x += kSelThreads) {
        const long long a = v[x];
        if ((a >> hi) != prefix) continue;
        const unsigned long long bin = ((unsigned long long)a >> lo) & (nbins - 1);
        if (bin == 0)
          zero_bin += a;
        else
          atomicAdd(&hist[bin], (unsigned long long)a);
      }
      zero_bin = block_sum_ll(zero_bin, red);
      if (tid == 0) {
        hist[0] = (unsigned long long)zero_bin;
        long long run = above;
        int d = 0;
        for (int bin = (int)nbins - 1; bin >= 0; --bin) {
          if (run + (long long)hist[bin] >= need) {
            d = bin;
            break;
          }
          run += (long long)hist[bin];
        }
        sh_state[0] = d;
        sh_state[1] = run;
      }
      __syncthreads();
      prefix = (prefix << width) | sh_state[0];
      above = sh_state[1];
      hi = lo;
      __syncthreads();
    }
    theta = prefix;
  }
  for (int x = tid; x < S; x += kSelThreads) {
    const long long a = v[x];
    keep[x] = (uint8_t)((a >= theta && a > 0) || x < band);
  }
}

template <int D, bool BF16>
hipError_t launch_sample_t(const void* q, const void* k, int32_t B, int32_t hq, int32_t hkv, int32_t S, int32_t row0,
                           int32_t n_rows, int32_t band, const uint8_t* skip_cols, bool lse_given, float scale,
                           float* row_lse, int64_t* diag, int64_t* vert, hipStream_t stream) {
  using E = typename SampleTypes<BF16>::E;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;
  const float scale_log2 = scale * kLog2e;
  const int nch = (n_rows + 31) / 32;
  if (!lse_given) {
    k_sample_lse<D, BF16><<<dim3((unsigned)(B * hq * nch)), dim3(512), 0, stream>>>(q, k, hq, hkv, S, row0, n_rows,
                                                                                    scale_log2, row_lse);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int ntile = (row0 + n_rows - 1) / 64 + 1;
  const size_t lds = 64 * KSTR * sizeof(E) + (64 + (size_t)n_rows + 63) * sizeof(unsigned long long);
  k_sample_acc<D, BF16><<<dim3((unsigned)(hq * ntile)), dim3(256), lds, stream>>>(
      q, k, B, hq, hkv, S, row0, n_rows, band, skip_cols, scale_log2, row_lse, reinterpret_cast<unsigned long long*>(diag),
      reinterpret_cast<unsigned long long*>(vert));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sample_scores(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                                int32_t head_dim, int32_t dtype, float scale, int32_t row0, int32_t n_rows,
                                int32_t band, const uint8_t* skip_cols, bool lse_given, float* row_lse, int64_t* diag,
                                int64_t* vert, hipStream_t stream) {
  if (dtype == SA_DTYPE_BF16)
    return head_dim == 64 ? launch_sample_t<64, true>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                      lse_given, scale, row_lse, diag, vert, stream)
                          : launch_sample_t<128, true>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                       lse_given, scale, row_lse, diag, vert, stream);
  return head_dim == 64 ? launch_sample_t<64, false>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols, lse_given,
                                                     scale, row_lse, diag, vert, stream)
                        : launch_sample_t<128, false>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                      lse_given, scale, row_lse, diag, vert, stream);
}

hipError_t launch_select(const int64_t* scores, int32_t n_heads, int32_t S, double alpha, int64_t t_all, int32_t band,
                         uint8_t* keep, hipStream_t stream) {
  k_select<<<dim3((unsigned)n_heads), dim3(kSelThreads), 0, stream>>>(reinterpret_cast<const long long*>(scores), S,
                                                                      alpha, (long long)t_all, band, keep);
  return hipGetLastError();
}

}  // namespace sa
