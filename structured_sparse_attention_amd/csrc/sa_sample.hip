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
// k_sample_part / k_sample_merge: the row LSE in two steps.  One workgroup of 8 waves
//   per (sequence, 256-key split, head) stages the split in LDS once; lane = query row,
//   S^T = K Q^T on MFMA, an online max/sum per row; the partial (max, sum) of every row
//   and split goes to the caller's workspace and is merged per row in split order.
// k_sample_acc: one workgroup of 4 waves per (64-key tile, head), heads of a kv group
//   adjacent; the tile is staged in LDS per sequence, the waves take 32-row chunks,
//   recompute the scores and add p = exp2(s - lse): diagonals summed per 32-row, 32-key
//   block through LDS (lane = diagonal, rows in order) and added with one int64 LDS
//   atomic per block and diagonal; verticals in registers, reduced across the lanes by a
//   butterfly and across the waves in a fixed order; one global int64 atomic per touched
//   pattern.
// k_select: one 1024-thread workgroup per head; the threshold is found by
//   a most-significant-digit radix search over the score bits (8-bit digits), each
//   pass a mass histogram of the scores inside the current bucket.
#include <type_traits>

#include <mutex>

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

// K rows [k0, k0 + nkeys) of one sequence and kv head into an LDS tile of stride KSTR (zeros past S)
template <int D, bool BF16, int NT>
__device__ inline void stage_keys(const typename SampleTypes<BF16>::E* K, int32_t S, int k0, int nkeys,
                                  typename SampleTypes<BF16>::E* Ks) {
  using E = typename SampleTypes<BF16>::E;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;
  constexpr int CH = D * (int)sizeof(E) / 16;  // 16-byte chunks per key row
  for (int x = threadIdx.x; x < nkeys * CH; x += NT) {
    const int r = x / CH, c = x % CH, j = k0 + r;
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
}

// S^T block of 32 keys (LDS rows kb*32 .. kb*32+31) against this lane's query row
template <int D, bool BF16>
__device__ inline sf32x16 score_block(const typename SampleTypes<BF16>::E* Ks, int kb, int r32, int g,
                                      const typename SampleTypes<BF16>::QF (&qf)[BF16 ? D / 16 : D / 2]) {
  constexpr int QS = BF16 ? D / 16 : D / 2;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;
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
  return acc;
}

// LSE pass 1: partial (max, sum) in the exp2 domain of every sampled row over one key
// split of kSplitKeys keys, staged once in LDS.  Grid: (sequence, key split, head),
// heads of one kv group adjacent so that the split is read from HBM about once.
constexpr int kSplitKeys = 256;

template <int D, bool BF16>
__global__ void __launch_bounds__(512) k_sample_part(const void* qv, const void* kv, int32_t hq, int32_t hkv,
                                                     int32_t S, int32_t row0, int32_t n_rows, int32_t nsplit,
                                                     float scale_log2, float2* part) {
  using E = typename SampleTypes<BF16>::E;
  using QF = typename SampleTypes<BF16>::QF;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* Ks = reinterpret_cast<E*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  const int h = blockIdx.x % hq;
  const int sp = (blockIdx.x / hq) % nsplit;
  const int b = blockIdx.x / (hq * nsplit);
  const int kvh = h / (hq / hkv);
  const int nch = (n_rows + 31) / 32;
  const int k0 = sp * kSplitKeys;
  const E* K = static_cast<const E*>(kv) + ((int64_t)b * hkv + kvh) * (int64_t)S * D;
  const E* Qh = static_cast<const E*>(qv) + ((int64_t)b * hq + h) * (int64_t)S * D;
  float2* out = part + ((int64_t)b * hq + h) * (int64_t)n_rows * nsplit;
  stage_keys<D, BF16, 512>(K, S, k0, kSplitKeys, Ks);
  __syncthreads();
  for (int ch = wave; ch < nch; ch += 8) {
    const int n = ch * 32 + r32;
    const bool row_ok = n < n_rows;
    const int i = row0 + (row_ok ? n : 0);
    const int chunk_last = row0 + ch * 32 + 31;
    float m = -INFINITY, l = 0.0f;
    if (chunk_last >= k0) {  // some row of the chunk reaches this split
      QF qf[BF16 ? D / 16 : D / 2];
      load_q_frags<D, BF16>(Qh + (int64_t)i * D, row_ok, g, qf);
      for (int kb = 0; kb < kSplitKeys / 32 && k0 + kb * 32 <= chunk_last; ++kb) {
        const sf32x16 acc = score_block<D, BF16>(Ks, kb, r32, g, qf);
        float x[16], tmax = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = k0 + kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
          x[v] = (row_ok && j <= i) ? acc[v] * scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, x[v]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));  // the row's other keys of the block sit in lane ^ 32
        const float mn = fmaxf(m, tmax);
        float p = 0.0f;
        if (mn != -INFINITY) {
#pragma unroll
          for (int v = 0; v < 16; ++v) p += __builtin_amdgcn_exp2f(x[v] - mn);
        }
        p += __shfl_xor(p, 32, 64);
        if (mn != -INFINITY) {
          l = (m == -INFINITY ? 0.0f : l * __builtin_amdgcn_exp2f(m - mn)) + p;
          m = mn;
        }
      }
    }
    if (g == 0 && row_ok) out[(int64_t)n * nsplit + sp] = make_float2(m, l);
  }
}

// LSE pass 2: the splits of each row merged (one wave per row; lanes take splits, then a
// fixed butterfly order), natural log out
__global__ void __launch_bounds__(256) k_sample_merge(const float2* part, int32_t rows_total, int32_t nsplit,
                                                      float* row_lse) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows_total) return;
  const float2* p = part + r * nsplit;
  float M = -INFINITY;
  for (int sp = lane; sp < nsplit; sp += 64) M = fmaxf(M, p[sp].x);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.0f;
  for (int sp = lane; sp < nsplit; sp += 64)
    if (p[sp].x != -INFINITY) L += p[sp].y * __builtin_amdgcn_exp2f(p[sp].x - M);
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o, 64);
  if (lane == 0) row_lse[r] = (M + __log2f(L)) * kLn2;
}

// v[0..31] summed over the 32 lanes that share lane & 32 (butterfly, fixed order);
// every lane of the half-wave ends with all 32 totals
__device__ inline void half_wave_sum(float (&v)[32]) {
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] += __shfl_xor(v[e], w, 64);
}

constexpr int kAccTiles = 16;  // 64-key tiles per workgroup of the accumulation pass

template <int D, bool BF16, bool DIAG, bool VERT>
// three waves per SIMD: the register budget that keeps the column pass free of spills (measured
// 10 % faster than the unconstrained two)
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_sample_acc(const void* qv, const void* kv, int32_t B, int32_t hq, int32_t hkv,
                                                    int32_t S, int32_t row0, int32_t n_rows, int32_t band,
                                                    const uint8_t* skip_cols, float scale_log2, const float* row_lse,
                                                    unsigned long long* diag_score, unsigned long long* vert_score) {
  using E = typename SampleTypes<BF16>::E;
  using QF = typename SampleTypes<BF16>::QF;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;  // LDS row stride of the key tile (elements)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* Ks = reinterpret_cast<E*>(smem);
  float* vpart = reinterpret_cast<float*>(smem + 64 * KSTR * sizeof(E));  // [4 waves][64 keys]
  unsigned long long* dacc = reinterpret_cast<unsigned long long*>(vpart + 4 * 64);  // diagonals r_base + x
  // per wave: the probabilities of one 32-row chunk against one 32-key half of the tile, [row][key]
  constexpr int kPS = 33;  // row stride (floats)
  __shared__ uint8_t skip_lds[kAccTiles * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  // heads fastest: the heads of one kv group read the same key tiles close together in time
  const int h = blockIdx.x % hq, grp = blockIdx.x / hq;
  const int kvh = h / (hq / hkv);
  const int last = row0 + n_rows - 1;
  const int c_first = grp * kAccTiles * 64;
  const int ntile = min(kAccTiles, (last - band - c_first) / 64 + 1);  // tiles some row reaches outside its window
  if (last - band < c_first) return;
  const int r_base = row0 - (c_first + kAccTiles * 64 - 1);  // diagonal of dacc[0]
  const int span = n_rows + kAccTiles * 64 - 1;
  float* pdiag = reinterpret_cast<float*>(dacc + (DIAG ? span : 0)) + wave * 32 * kPS;
  const int nch = (n_rows + 31) / 32;
  if constexpr (DIAG)
    for (int x = tid; x < span; x += 256) dacc[x] = 0ull;
  for (int x = tid; x < kAccTiles * 64; x += 256) {
    const int c = c_first + x;
    skip_lds[x] = (skip_cols && c < S) ? skip_cols[(int64_t)h * S + c] : 0;
  }
  unsigned long long* dg = DIAG ? diag_score + (int64_t)h * S : nullptr;
  unsigned long long* vt = VERT ? vert_score + (int64_t)h * S : nullptr;
  // a wave with one chunk and one sequence keeps its query fragments across the tiles
  const bool q_fixed = B == 1 && nch <= 4;
  QF qf[BF16 ? D / 16 : D / 2];
  float lse2 = 0.0f;
  auto load_q = [&](int b, int ch) {
    const int n = ch * 32 + r32;
    const bool row_ok = n < n_rows;
    const int i = row0 + (row_ok ? n : 0);
    load_q_frags<D, BF16>(static_cast<const E*>(qv) + (((int64_t)b * hq + h) * S + i) * (int64_t)D, row_ok, g, qf);
    lse2 = row_ok ? row_lse[((int64_t)b * hq + h) * n_rows + n] * kLog2e : 0.0f;
  };
  if (q_fixed && wave < nch) load_q(0, wave);

  for (int t = 0; t < ntile; ++t) {
    const int c0 = c_first + t * 64;
    float vacc[32];  // entry kb * 16 + v: key kb*32 + 8(v/4) + 4g + v%4 of the tile
#pragma unroll
    for (int x = 0; x < 32; ++x) vacc[x] = 0.0f;
    for (int b = 0; b < B; ++b) {
      __syncthreads();
      stage_keys<D, BF16, 256>(static_cast<const E*>(kv) + ((int64_t)b * hkv + kvh) * (int64_t)S * D, S, c0, 64, Ks);
      __syncthreads();
      for (int ch = wave; ch < nch; ch += 4) {
        if (row0 + ch * 32 + 31 < c0 + band) continue;  // no row of the chunk reaches the tile outside its window
        if (!q_fixed) load_q(b, ch);
        const int n = ch * 32 + r32;
        const bool row_ok = n < n_rows;
        const int i = row0 + (row_ok ? n : 0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const sf32x16 acc = score_block<D, BF16>(Ks, kb, r32, g, qf);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int jt = kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
            const int j = c0 + jt;
            const bool ok = row_ok && j <= i - band && !skip_lds[t * 64 + jt];
            const float p = ok ? __builtin_amdgcn_exp2f(acc[v] * scale_log2 - lse2) : 0.0f;
            if constexpr (VERT) vacc[kb * 16 + v] += p;
            if constexpr (DIAG) pdiag[r32 * kPS + (jt - kb * 32)] = p;
          }
          if constexpr (DIAG) {
            // diagonal sums of the 32 x 32 block: lane x takes diagonal (row - key) = x - 31, its rows
            // in ascending order, then one fixed-point value and one LDS atomic per diagonal
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's block is in LDS
            if (lane < 63) {
              const int dl = lane - 31;
              float sum = 0.0f;
              for (int r = max(0, dl); r <= min(31, 31 + dl); ++r) sum += pdiag[r * kPS + (r - dl)];
              const unsigned long long fx = (unsigned long long)__double2ll_rn((double)sum * kFixUnit);
              if (fx) atomicAdd(&dacc[(row0 + ch * 32 - c0 - kb * 32) + dl - r_base], fx);
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next block overwrites it
          }
        }
      }
    }
    // verticals of this tile: the lanes' partial sums reduced over the 32 rows of each
    // half-wave, then over the waves in a fixed order, then rounded once to fixed point
    if constexpr (!VERT) continue;
    half_wave_sum(vacc);
    if (r32 == 0) {
#pragma unroll
      for (int e = 0; e < 32; ++e) vpart[wave * 64 + (e >> 4) * 32 + 8 * ((e & 15) >> 2) + 4 * g + (e & 3)] = vacc[e];
    }
    __syncthreads();
    if (tid < 64 && c0 + tid < S) {
      const float vs = ((vpart[tid] + vpart[64 + tid]) + vpart[128 + tid]) + vpart[192 + tid];
      const unsigned long long fx = (unsigned long long)__double2ll_rn((double)vs * kFixUnit);
      if (fx) atomicAdd(&vt[c0 + tid], fx);
    }
  }
  if constexpr (DIAG) {
    __syncthreads();
    for (int x = tid; x < span; x += 256) {
      const int r = r_base + x;
      if (dacc[x] && r >= 0 && r < S) atomicAdd(&dg[r], dacc[x]);
    }
  }
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

int32_t sample_splits(int32_t row0, int32_t n_rows) { return (row0 + n_rows - 1) / kSplitKeys + 1; }

template <int D, bool BF16>
hipError_t launch_sample_t(const void* q, const void* k, int32_t B, int32_t hq, int32_t hkv, int32_t S, int32_t row0,
                           int32_t n_rows, int32_t band, const uint8_t* skip_cols, bool lse_given, float scale,
                           float* row_lse, void* workspace, int64_t* diag, int64_t* vert, hipStream_t stream) {
  using E = typename SampleTypes<BF16>::E;
  constexpr int KSTR = BF16 ? D + 8 : D + 1;
  const float scale_log2 = scale * kLog2e;
  if (!lse_given) {
    const int32_t nsplit = sample_splits(row0, n_rows);
    float2* part = static_cast<float2*>(workspace);
    const size_t lds = (size_t)kSplitKeys * KSTR * sizeof(E);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sample_part<D, BF16>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    k_sample_part<D, BF16><<<dim3((unsigned)((int64_t)B * nsplit * hq)), dim3(512), lds, stream>>>(
        q, k, hq, hkv, S, row0, n_rows, nsplit, scale_log2, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)B * hq * n_rows;
    k_sample_merge<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(part, (int32_t)rows, nsplit, row_lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int ngrp = (row0 + n_rows - 1) / (kAccTiles * 64) + 1;
  const size_t lds = 64 * KSTR * sizeof(E) + 4 * 64 * sizeof(float) +
                     (diag ? ((size_t)n_rows + kAccTiles * 64 - 1) * sizeof(unsigned long long) +
                                 4 * 32 * 33 * sizeof(float)
                           : 0);
  auto kern = diag ? (vert ? k_sample_acc<D, BF16, true, true> : k_sample_acc<D, BF16, true, false>)
                   : k_sample_acc<D, BF16, false, true>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)(hq * ngrp)), dim3(256), lds, stream>>>(q, k, B, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                                scale_log2, row_lse,
                                                                reinterpret_cast<unsigned long long*>(diag),
                                                                reinterpret_cast<unsigned long long*>(vert));
  return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate: the per-split row statistics of the LSE
// pass in a static device array, one copy per GPU, held until the process ends.  Its
// device address is taken once per device (hipGetSymbolAddress with that device
// current) and passed to the kernels like a caller's workspace; the array's name is a
// host-side stand-in and is never handed to a kernel.
static __device__ __align__(256) unsigned char scratch[kSampleStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t sample_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t sample_workspace_bytes(int32_t batch, int32_t hq, int32_t row0, int32_t n_rows) {
  return (size_t)batch * hq * n_rows * sample_splits(row0, n_rows) * sizeof(float2);
}

hipError_t launch_sample_scores(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                                int32_t head_dim, int32_t dtype, float scale, int32_t row0, int32_t n_rows,
                                int32_t band, const uint8_t* skip_cols, bool lse_given, float* row_lse, void* workspace,
                                int64_t* diag, int64_t* vert, hipStream_t stream) {
  if (dtype == SA_DTYPE_BF16)
    return head_dim == 64 ? launch_sample_t<64, true>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                      lse_given, scale, row_lse, workspace, diag, vert, stream)
                          : launch_sample_t<128, true>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                       lse_given, scale, row_lse, workspace, diag, vert, stream);
  return head_dim == 64 ? launch_sample_t<64, false>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols, lse_given,
                                                     scale, row_lse, workspace, diag, vert, stream)
                        : launch_sample_t<128, false>(q, k, batch, hq, hkv, S, row0, n_rows, band, skip_cols,
                                                      lse_given, scale, row_lse, workspace, diag, vert, stream);
}

hipError_t launch_select(const int64_t* scores, int32_t n_heads, int32_t S, double alpha, int64_t t_all, int32_t band,
                         uint8_t* keep, hipStream_t stream) {
  k_select<<<dim3((unsigned)n_heads), dim3(kSelThreads), 0, stream>>>(reinterpret_cast<const long long*>(scores), S,
                                                                      alpha, (long long)t_all, band, keep);
  return hipGetLastError();
}

}  // namespace sa
