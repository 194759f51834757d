// sa_index.hip -- pattern descriptor -> canonical sparse index, on the device (gfx950).
//
// The pages give the patterns (Pith review of "DAM: Dynamic Attention Mask for
// Long-Context Large Language Model Inference Acceleration", "What carries the
// argument": diagonals j = i - r, verticals j = c with i >= c; SeerAttention
// abstract: 64 x 64 blocks; AnchorAttention abstract: stripe granularity) but no
// index format.  The index here is this library's: for each (head, row block) the
// key columns that the diagonals touch (U, as maximal intervals) and the column
// part X (verticals, blocks, stripe lists) split into X & U and X \ U.  Its exact
// definition is in include/sa.h.
//
// Work layout: one 256-thread workgroup per (head, row block).  The workgroup
// builds two bitmaps over key columns [0, b1] in LDS -- X and U -- with one word
// per thread per step (blocks, interval fills) and LDS atomics (vertical and stripe
// lists).  Everything after that is word-parallel: popcounts give the counts,
// a block-wide scan gives write positions, and segment starts/ends are the rising
// and falling edges of U.  The pass runs twice per build: counting (then a device
// scan turns counts into offsets) and filling.  HBM traffic: the stripe lists and
// block-mask rows in, the index out; everything else stays in LDS.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// number of elements <= x in the sorted array a[0, n)
__device__ inline int32_t upper_bound_i32(const int32_t* a, int32_t n, int32_t x) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// bits [a, b] of a 32-bit word, 0 <= a <= b <= 31
__device__ inline uint32_t bit_range(int a, int b) {
  uint32_t hi = (b == 31) ? 0xffffffffu : ((1u << (b + 1)) - 1u);
  return hi & ~((1u << a) - 1u);
}

// ---------------------------------------------------------------------------
// Runs of D_h (maximal runs of consecutive offsets), validation of the D and C
// lists, and reset of pair_count / status.  A single workgroup: heads are few.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_runs(sa_pattern_desc d, sa_index ix, int32_t validate) {
  const int tid = threadIdx.x;
  if (tid == 0) ix.status[0] = 0;
  __syncthreads();
  for (int h = tid; h < d.n_heads; h += kThreads) {
    ix.pair_count[h] = 0;
    const int32_t p0 = d.diag_ptr[h], p1 = d.diag_ptr[h + 1];
    int32_t n = 0, prev = -1;
    bool bad = false;
    for (int32_t p = p0; p < p1; ++p) {
      int32_t r = d.diag_off[p];
      if (validate && (r < 0 || r >= d.S || r <= prev)) bad = true;
      if (p == p0 || r != prev + 1) ++n;
      prev = r;
    }
    if (validate) {
      int32_t pv = -1;
      for (int32_t p = d.vert_ptr[h]; p < d.vert_ptr[h + 1]; ++p) {
        int32_t c = d.vert_col[p];
        if (c < 0 || c >= d.S || c <= pv) bad = true;
        pv = c;
      }
    }
    if (bad) atomicOr(ix.status, SA_STATUS_DESC_INVALID);
    ix.run_ptr[h + 1] = n;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    ix.run_ptr[0] = 0;
    for (int h = 0; h < d.n_heads; ++h) {
      acc += ix.run_ptr[h + 1];
      ix.run_ptr[h + 1] = acc;
    }
  }
  __syncthreads();
  if (ix.run_lo == nullptr || ix.run_hi == nullptr) return;
  for (int h = tid; h < d.n_heads; h += kThreads) {
    const int32_t p0 = d.diag_ptr[h], p1 = d.diag_ptr[h + 1];
    int64_t out = ix.run_ptr[h];
    int32_t p = p0;
    while (p < p1) {
      int32_t lo = d.diag_off[p], hi = lo;
      while (p + 1 < p1 && d.diag_off[p + 1] == hi + 1) { ++p; ++hi; }
      if (out < ix.capacity.n_runs) {
        ix.run_lo[out] = lo;
        ix.run_hi[out] = hi;
      } else {
        atomicOr(ix.status, SA_STATUS_OVERFLOW);
      }
      ++out;
      ++p;
    }
  }
}

// Block-wide exclusive scan of four counters; returns the totals in tot[].
__device__ inline void block_scan4(int32_t v[4], int32_t tot[4], int32_t* sh /* [kWaves*4] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t inc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int32_t x = v[c];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    inc[c] = x;
  }
  if (lane == 63) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sh[wave * 4 + c] = inc[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    int32_t before = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
      int32_t t = sh[w * 4 + c];
      if (w < wave) before += t;
      all += t;
    }
    v[c] = before + inc[c] - v[c];
    tot[c] = all;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Per (head, row block): build X and U bitmaps, then count (fill = 0) or write
// (fill = 1) segments, in-segment columns and gathered columns.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_items(sa_pattern_desc d, sa_index ix, int32_t fill, int32_t validate) {
  extern __shared__ uint32_t lds[];
  __shared__ int32_t scan_sh[kWaves * 4];
  __shared__ long long red_sh[kWaves * 4];

  const int tid = threadIdx.x;
  const int32_t S = d.S, BM = ix.row_block, nb = ix.n_row_blocks;
  const int64_t it = blockIdx.x;
  const int32_t h = (int32_t)(it / nb), rb = (int32_t)(it % nb);
  const int32_t b0 = rb * BM, b1 = min(S, b0 + BM) - 1;
  const int32_t nw = (b1 >> 5) + 1;          // words covering columns [0, b1]
  const int32_t nw_alloc = ((S - 1) >> 5) + 1;
  uint32_t* X = lds;
  uint32_t* U = lds + nw_alloc;

  // --- X from the block row, U cleared
  const uint8_t* brow = nullptr;
  int64_t nbq = 0;
  if (d.block_mask != nullptr) {
    nbq = cdiv64(S, d.block_size);
    brow = d.block_mask + ((int64_t)h * nbq + b0 / d.block_size) * nbq;
  }
  for (int32_t w = tid; w < nw; w += kThreads) {
    uint32_t x = 0;
    if (brow != nullptr && brow[(w * 32) / d.block_size]) x = 0xffffffffu;
    if (w == nw - 1) x &= bit_range(0, b1 & 31);
    X[w] = x;
    U[w] = 0;
  }
  __syncthreads();

  // --- verticals and stripe columns into X
  {
    const int32_t p0 = d.vert_ptr[h], p1 = d.vert_ptr[h + 1];
    for (int32_t p = p0 + tid; p < p1; p += kThreads) {
      int32_t c = d.vert_col[p];
      if (c >= 0 && c <= b1) atomicOr(&X[c >> 5], 1u << (c & 31));
    }
  }
  if (d.stripe_ptr != nullptr) {
    const int64_t nst = cdiv64(S, d.stripe_rows);
    const int64_t t = b0 / d.stripe_rows;
    const int64_t p0 = d.stripe_ptr[h * nst + t], p1 = d.stripe_ptr[h * nst + t + 1];
    bool bad = false;
    for (int64_t p = p0 + tid; p < p1; p += kThreads) {
      int32_t c = d.stripe_col[p];
      if (validate && (c < 0 || c >= S || (p > p0 && d.stripe_col[p - 1] >= c))) bad = true;
      if (c >= 0 && c <= b1) atomicOr(&X[c >> 5], 1u << (c & 31));
    }
    if (bad) atomicOr(ix.status, SA_STATUS_DESC_INVALID);
  }
  // --- U: columns i - r for i in [b0, b1] and r in a run [lo, hi] of D_h: [b0 - hi, b1 - lo], clipped
  // to [0, b1].  A thread that holds the first offset of a run finds the run's end by binary search:
  // diag_off[q] - q is non-decreasing and constant exactly along a run.
  {
    const int32_t p0 = d.diag_ptr[h], p1 = d.diag_ptr[h + 1];
    for (int32_t p = p0 + tid; p < p1; p += kThreads) {
      const int32_t lo = d.diag_off[p];
      if (p > p0 && d.diag_off[p - 1] == lo - 1) continue;  // not the first offset of a run
      if (lo > b1) continue;
      int32_t qa = p, qb = p1 - 1;
      while (qa < qb) {
        const int32_t mid = (qa + qb + 1) >> 1;
        if (d.diag_off[mid] - mid == lo - p) qa = mid;
        else qb = mid - 1;
      }
      const int32_t hi = d.diag_off[qa];
      const int32_t a = max(0, b0 - hi), e = min(b1, b1 - lo);
      for (int32_t w = a >> 5; a <= e && w <= (e >> 5); ++w) {
        const int32_t ba = max(a, w * 32) - w * 32, be = min(e, w * 32 + 31) - w * 32;
        atomicOr(&U[w], bit_range(ba, be));
      }
    }
  }
  __syncthreads();

  const int32_t* Dh = d.diag_off + d.diag_ptr[h];
  const int32_t nD = d.diag_ptr[h + 1] - d.diag_ptr[h];

  if (!fill) {
    int64_t n_seg = 0, n_in = 0, n_out = 0, pairs = 0;
    for (int32_t w = tid; w < nw; w += kThreads) {
      const uint32_t u = U[w], x = X[w];
      const uint32_t prev_msb = (w > 0) ? (U[w - 1] >> 31) : 0u;
      n_seg += __popc(u & ~((u << 1) | prev_msb));
      uint32_t in = x & u, out = x & ~u;
      n_in += __popc(in);
      n_out += __popc(out);
      // gathered columns: rows max(j, b0) .. b1, all retained
      if (w * 32 + 31 < b0) {
        pairs += (int64_t)__popc(out) * (int64_t)(b1 - b0 + 1);
      } else {
        while (out) {
          int bit = __ffs(out) - 1;
          out &= out - 1;
          int32_t j = w * 32 + bit;
          pairs += b1 - max(j, b0) + 1;
        }
      }
      // in-segment columns of X: every causal row minus the rows whose offset is a diagonal
      while (in) {
        int bit = __ffs(in) - 1;
        in &= in - 1;
        int32_t j = w * 32 + bit;
        int32_t a = max(j, b0);
        int32_t dcount = upper_bound_i32(Dh, nD, b1 - j) - upper_bound_i32(Dh, nD, a - j - 1);
        pairs += (b1 - a + 1) - dcount;
      }
    }
    // diagonal pairs of each row: offsets r in D_h with r <= i
    for (int32_t i = b0 + tid; i <= b1; i += kThreads) pairs += upper_bound_i32(Dh, nD, i);

    // block reduction of the four counters
    const int lane = tid & 63, wave = tid >> 6;
    long long vals[4] = {(long long)n_seg, (long long)n_in, (long long)n_out, (long long)pairs};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      long long x = vals[c];
      for (int o = 32; o > 0; o >>= 1) x += __shfl_down(x, o, 64);
      if (lane == 0) red_sh[wave * 4 + c] = x;
    }
    __syncthreads();
    if (tid == 0) {
      long long t[4] = {0, 0, 0, 0};
      for (int w = 0; w < kWaves; ++w)
        for (int c = 0; c < 4; ++c) t[c] += red_sh[w * 4 + c];
      ix.seg_ptr[it + 1] = t[0];
      ix.bcol_ptr[it + 1] = t[1];
      ix.col_ptr[it + 1] = t[2];
      if (it == 0) {
        ix.seg_ptr[0] = 0;
        ix.bcol_ptr[0] = 0;
        ix.col_ptr[0] = 0;
      }
      atomicAdd((unsigned long long*)&ix.pair_count[h], (unsigned long long)t[3]);
    }
    return;
  }

  // --- fill: word-per-thread chunks, block scan for write positions
  int64_t base_rise = ix.seg_ptr[it], base_fall = ix.seg_ptr[it], base_in = ix.bcol_ptr[it],
          base_out = ix.col_ptr[it];
  bool overflow = false;
  for (int32_t w0 = 0; w0 < nw; w0 += kThreads) {
    const int32_t w = w0 + tid;
    uint32_t rise = 0, fall = 0, in = 0, out = 0;
    if (w < nw) {
      const uint32_t u = U[w], x = X[w];
      const uint32_t prev_msb = (w > 0) ? (U[w - 1] >> 31) : 0u;
      const uint32_t next_lsb = (w + 1 < nw) ? (U[w + 1] & 1u) : 0u;
      rise = u & ~((u << 1) | prev_msb);
      fall = u & ~((u >> 1) | (next_lsb << 31));
      in = x & u;
      out = x & ~u;
    }
    int32_t v[4] = {(int32_t)__popc(rise), (int32_t)__popc(fall), (int32_t)__popc(in), (int32_t)__popc(out)};
    int32_t tot[4];
    block_scan4(v, tot, scan_sh);
    int64_t pr = base_rise + v[0], pf = base_fall + v[1], pi = base_in + v[2], po = base_out + v[3];
    while (rise) {
      int bit = __ffs(rise) - 1;
      rise &= rise - 1;
      if (pr < ix.capacity.n_segs) ix.seg_lo[pr] = w * 32 + bit; else overflow = true;
      ++pr;
    }
    while (fall) {
      int bit = __ffs(fall) - 1;
      fall &= fall - 1;
      if (pf < ix.capacity.n_segs) ix.seg_hi[pf] = w * 32 + bit; else overflow = true;
      ++pf;
    }
    while (in) {
      int bit = __ffs(in) - 1;
      in &= in - 1;
      if (pi < ix.capacity.n_bcols) ix.bcol_idx[pi] = w * 32 + bit; else overflow = true;
      ++pi;
    }
    while (out) {
      int bit = __ffs(out) - 1;
      out &= out - 1;
      if (po < ix.capacity.n_cols) ix.col_idx[po] = w * 32 + bit; else overflow = true;
      ++po;
    }
    base_rise += tot[0];
    base_fall += tot[1];
    base_in += tot[2];
    base_out += tot[3];
  }
  if (overflow) atomicOr(ix.status, SA_STATUS_OVERFLOW);
}

// ---------------------------------------------------------------------------
// Diagonal offsets as a bitmap: one thread per 32-bit word; the word's offsets
// [32w, 32w + 31] are a contiguous slice of the sorted list, found by binary search.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_dbits(sa_pattern_desc d, uint32_t* dbits, int32_t nwords) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (int64_t)d.n_heads * nwords) return;
  const int32_t h = (int32_t)(gid / nwords), w = (int32_t)(gid % nwords);
  const int32_t* D = d.diag_off + d.diag_ptr[h];
  const int32_t n = d.diag_ptr[h + 1] - d.diag_ptr[h];
  int32_t p = upper_bound_i32(D, n, w * 32 - 1);  // first offset >= 32w
  uint32_t bits = 0;
  for (; p < n && D[p] < w * 32 + 32; ++p)
    if (D[p] >= w * 32) bits |= 1u << (D[p] - w * 32);
  dbits[gid] = bits;
}

// ---------------------------------------------------------------------------
// In-place inclusive scan of entries 1..n of the three item pointer arrays
// (entry 0 is 0), so that ptr[it] is the first element of item it.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads) k_scan(int64_t* a0, int64_t* a1, int64_t* a2, int64_t n) {
  __shared__ long long part[kScanThreads];
  int64_t* arrs[3] = {a0, a1, a2};
  const int tid = threadIdx.x;
  const int64_t per = cdiv64(n, kScanThreads);
  const int64_t s = 1 + tid * per, e = min(n + 1, s + per);
  for (int c = 0; c < 3; ++c) {
    int64_t* a = arrs[c];
    long long local = 0;
    for (int64_t p = s; p < e; ++p) local += a[p];
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < kScanThreads; o <<= 1) {
      long long y = (tid >= o) ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += y;
      __syncthreads();
    }
    long long run = part[tid] - local;
    for (int64_t p = s; p < e; ++p) {
      run += a[p];
      a[p] = run;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_index_runs(const sa_pattern_desc& d, const sa_index& ix, int32_t validate, hipStream_t stream) {
  hipLaunchKernelGGL(k_runs, dim3(1), dim3(kThreads), 0, stream, d, ix, validate);
  return hipGetLastError();
}

hipError_t launch_index_items(const sa_pattern_desc& d, const sa_index& ix, int32_t fill, int32_t validate,
                              hipStream_t stream) {
  const int64_t items = (int64_t)ix.n_heads * ix.n_row_blocks;
  const size_t lds = 2 * sizeof(uint32_t) * (size_t)(((d.S - 1) >> 5) + 1);
  hipLaunchKernelGGL(k_items, dim3((unsigned)items), dim3(kThreads), lds, stream, d, ix, fill, validate);
  return hipGetLastError();
}

hipError_t launch_index_dbits(const sa_pattern_desc& d, const sa_index& ix, hipStream_t stream) {
  const int32_t nwords = ((d.S - 1) >> 5) + 1;
  const int64_t total = (int64_t)d.n_heads * nwords;
  hipLaunchKernelGGL(k_dbits, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream, d,
                     ix.dbits, nwords);
  return hipGetLastError();
}

hipError_t launch_index_scan(const sa_index& ix, hipStream_t stream) {
  const int64_t items = (int64_t)ix.n_heads * ix.n_row_blocks;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, stream, ix.seg_ptr, ix.bcol_ptr, ix.col_ptr, items);
  return hipGetLastError();
}

}  // namespace sa
