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
// A build is nine launches, all on one stream:
//   k_heads         one workgroup per head: validation of D and C, the run count of D,
//                   reset of status
//   k_items_lists   one wave per (head, row block), count pass: classifies the item and
//                   counts the items that need no bitmap (block columns only, a stripe list
//                   only, or diagonals and verticals)
//   k_items         count pass of the other items (bitmaps in LDS)
//   k_scan_local  |
//   k_scan_offset | exclusive scans of the per-item counts and of the per-head run
//   k_scan_fix    | counts (three passes, no workspace: the arrays are scanned in place)
//   k_items_lists   fill pass
//   k_items         fill pass
//   k_heads_fill    one workgroup per head: pair_count, the D bitmap (dbits), the runs of D
// Between the passes each item keeps its kind and retained-pair count in its slot of
// dbits, which k_heads_fill overwrites with the bitmap at the end.
// Bitmap path: X and U over key columns [0, b1] in LDS, with one word per thread per
// step (blocks, interval fills) and LDS atomics (vertical and stripe lists);
// everything after that is word-parallel: popcounts give the counts, a block-wide scan
// gives write positions, and segment starts/ends are the rising and falling edges of U.
// Without bitmaps: block columns are whole blocks in order; the columns <= b1 of a
// sorted stripe list are a prefix of it; a vertical c lies in U iff some offset of D
// falls in [max(b0, c) - c, b1 - c]; the segments of U are the merged column intervals
// of the runs of D.  The head's diagonal offsets are staged in LDS (when they fit) for
// the binary searches.  HBM traffic: the descriptor lists and block-mask rows in, the
// index out.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kDsh = 2048;                      // diagonal offsets of one head staged in LDS (also the fill's stage)
constexpr int kScanPer = 16;                    // scan entries per thread
constexpr int kScanChunk = kThreads * kScanPer; // scan entries per workgroup
constexpr int32_t kBadHead = 1 << 30;           // run_ptr marker from k_heads to k_scan_fix
constexpr size_t kDefaultLds = 65536;           // dynamic LDS usable without raising the function's limit

// number of elements <= x in the sorted array a[0, n) (a may point to LDS or global memory)
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

// true iff offset r does not continue the run of its predecessor (wrap-safe for invalid lists)
__device__ inline bool starts_run(int32_t r, int32_t prev) { return (uint32_t)r != (uint32_t)prev + 1u; }

// a[i] for lo <= i < hi, else `fill`; [lo, hi) must be a non-empty range of valid indices.  The load
// itself is unconditional, from the index clamped into [lo, hi), so that a batch of these calls
// leaves every load in flight at once (a load under a branch is waited for before the branch joins:
// one round trip per element).
template <typename T, typename I>
__device__ inline T load_in(const T* a, I i, I lo, I hi, T fill) {
  const T x = a[i < lo ? lo : (i < hi ? i : hi - 1)];
  return (i >= lo && i < hi) ? x : fill;
}

// Workgroup-wide exclusive scan of one value per thread; *total receives the sum.  Contains
// two barriers, so every read a thread made before the call precedes every write after it.
template <typename T>
__device__ inline T block_exscan(T x, T* total, T* sh /* [kWaves] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  T before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    T t = sh[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

template <typename T>
__device__ inline T block_sum(T x, T* sh /* [kWaves] */) {
  T tot;
  block_exscan<T>(x, &tot, sh);
  return tot;
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
// Per head, before the count: reset status and run_ptr[0] (once); validate the D
// and C lists; count the maximal runs of D into run_ptr[h + 1] (kBadHead marks an
// invalid head until k_scan_fix folds it into status).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_heads(sa_pattern_desc d, sa_index ix, int32_t validate) {
  __shared__ int32_t red[kWaves];
  const int tid = threadIdx.x;
  const int32_t h = blockIdx.x, S = d.S;
  if (h == 0 && tid == 0) {
    ix.status[0] = 0;
    ix.run_ptr[0] = 0;
  }
  const int32_t p0 = d.diag_ptr[h], p1 = d.diag_ptr[h + 1];
  int32_t runs = 0, bad = 0;
  for (int32_t pb = p0; pb < p1; pb += 4 * kThreads) {
    int32_t r[4], prev[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t p = pb + u * kThreads + tid;
      r[u] = load_in<int32_t, int32_t>(d.diag_off, p, p0, p1, 0);
      prev[u] = load_in<int32_t, int32_t>(d.diag_off, p - 1, p0, p1, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t p = pb + u * kThreads + tid;
      if (p >= p1) continue;
      if (validate && (r[u] < 0 || r[u] >= S || (p > p0 && r[u] <= prev[u]))) bad = 1;
      if (p == p0 || starts_run(r[u], prev[u])) ++runs;
    }
  }
  if (validate) {
    const int32_t q0 = d.vert_ptr[h], q1 = d.vert_ptr[h + 1];
    for (int32_t p = q0 + tid; p < q1; p += kThreads) {
      const int32_t c = d.vert_col[p];
      if (c < 0 || c >= S || (p > q0 && d.vert_col[p - 1] >= c)) bad = 1;
    }
  }
  runs = block_sum<int32_t>(runs, red);
  bad = block_sum<int32_t>(bad, red);
  if (tid == 0) ix.run_ptr[h + 1] = runs | (bad ? kBadHead : 0);
}

// Launch constants of the item kernels, computed on the host (32-bit: S <= 262144, items < 2^31).
struct ItemConsts {
  int32_t nbq;        // block-mask row length, ceil(S / block_size) (0 without a block mask)
  int32_t rb_per_br;  // row blocks per block row, block_size / BM
  int32_t wpb_shift;  // log2(block_size / 32) when that is a power of two, else -1
  int32_t wpb;        // block_size / 32
  int32_t bs;         // block_size (a multiple of 64)
  int32_t nst;        // stripes per head, ceil(S / stripe_rows) (0 without stripes)
  int32_t rb_per_st;  // row blocks per stripe, stripe_rows / BM
  int32_t dcap;       // diagonal offsets that fit the LDS staging area
  int32_t nwords;     // ceil(S / 32): length of one dbits row
};

// How an item is built.  The count pass of k_items_lists decides it and keeps it in the two top
// bits of the item's scratch slot dbits[h][rb] (the low bits hold its retained-pair count); every
// later item pass reads it from there.
//   kKindBlocks   only block-mask columns (no diagonal, vertical or stripe list)
//   kKindStripes  only a stripe list
//   kKindLists    diagonals and verticals, no block or stripe column, the diagonals fit in LDS
//   kKindGeneral  anything else: the bitmap path of k_items
constexpr uint32_t kKindBlocks = 0, kKindStripes = 1, kKindLists = 2, kKindGeneral = 3;
constexpr int kKindShift = 30;
constexpr uint32_t kPairsMask = (1u << kKindShift) - 1u;  // an item holds at most BM * S <= 2^25 pairs

struct Item {
  int32_t it, h, rb, b0, b1, nw;
  int32_t nD, vp0, vp1;
  int64_t sp0, sp1;
  const int32_t* D;     // the head's diagonal offsets (global)
  const uint8_t* brow;  // the block row of this row block, or null
  int32_t cb1;          // block column that holds column b1
};

// Values the whole wave shares, loaded through the vector memory path, moved to scalar registers.
__device__ inline int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// `it` must be the same for the whole wave.
__device__ inline Item load_item(const sa_pattern_desc& d, const sa_index& ix, const ItemConsts& kc, int32_t it) {
  Item m;
  const int32_t S = d.S, BM = ix.row_block, nb = ix.n_row_blocks;
  m.it = it;
  m.h = m.it / nb;
  m.rb = m.it - m.h * nb;
  m.b0 = m.rb * BM;
  m.b1 = min(S, m.b0 + BM) - 1;
  m.nw = (m.b1 >> 5) + 1;
  // every list bound this item needs, loaded together
  const int32_t dp0 = d.diag_ptr[m.h], dp1 = d.diag_ptr[m.h + 1];
  m.vp0 = d.vert_ptr[m.h];
  m.vp1 = d.vert_ptr[m.h + 1];
  m.sp0 = m.sp1 = 0;
  if (d.stripe_ptr != nullptr) {
    const int64_t st = (int64_t)m.h * kc.nst + m.rb / kc.rb_per_st;
    m.sp0 = d.stripe_ptr[st];
    m.sp1 = d.stripe_ptr[st + 1];
  }
  // the item is the same for the whole wave: its bounds go to scalar registers
  m.vp0 = uni(m.vp0);
  m.vp1 = uni(m.vp1);
  m.sp0 = uni64(m.sp0);
  m.sp1 = uni64(m.sp1);
  m.nD = uni(dp1 - dp0);
  m.D = d.diag_off + uni(dp0);
  m.brow = nullptr;
  m.cb1 = 0;
  if (d.block_mask != nullptr) {
    m.brow = d.block_mask + ((int64_t)m.h * kc.nbq + m.rb / kc.rb_per_br) * kc.nbq;
    m.cb1 = kc.wpb_shift >= 0 ? ((m.b1 >> 5) >> kc.wpb_shift) : (m.b1 >> 5) / kc.wpb;
  }
  return m;
}

__device__ inline uint32_t* scratch_slot(const sa_index& ix, const ItemConsts& kc, const Item& m) {
  return ix.dbits + (int64_t)m.h * kc.nwords + m.rb;
}

// Workgroup reduction of the four item counters; thread 0 stores them and the scratch slot.
__device__ inline void store_counts(const sa_index& ix, const ItemConsts& kc, const Item& m, long long cnt[4],
                                    uint32_t kind, long long* red_sh /* [kWaves * 4] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    long long x = cnt[c];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_down(x, o, 64);
    if (lane == 0) red_sh[wave * 4 + c] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long t[4] = {0, 0, 0, 0};
    for (int w = 0; w < kWaves; ++w)
      for (int c = 0; c < 4; ++c) t[c] += red_sh[w * 4 + c];
    ix.seg_ptr[m.it + 1] = t[0];
    ix.bcol_ptr[m.it + 1] = t[1];
    ix.col_ptr[m.it + 1] = t[2];
    *scratch_slot(ix, kc, m) = ((uint32_t)t[3] & kPairsMask) | (kind << kKindShift);
  }
}

// Retained pairs of gathered columns c0..c1 (all rows max(j, b0) .. b1 retained), 0 <= c0 <= c1 <= b1.
__device__ inline long long column_pairs(int32_t c0, int32_t c1, int32_t b0, int32_t b1) {
  long long p = 0;
  const int32_t below = min(c1, b0 - 1);  // columns under the row block: every row
  if (below >= c0) p += (long long)(below - c0 + 1) * (b1 - b0 + 1);
  const int32_t a = max(c0, b0);          // columns inside: rows j .. b1
  if (c1 >= a) {
    const long long n = c1 - a + 1;
    p += n * (b1 + 1) - (long long)(a + c1) * n / 2;
  }
  return p;
}

// Number of entries <= x of the sorted global array a[0, n), found by one wave: each round probes
// 64 evenly spaced entries and keeps the gap between the last probe <= x and the next one (a
// round per factor of 64 in n).  Every lane returns the result.
__device__ inline int64_t wave_upper_bound(const int32_t* a, int64_t n, int32_t x) {
  const int lane = threadIdx.x & 63;
  int64_t lo = 0, hi = n;  // invariant: a[i] <= x for i < lo, a[i] > x for i >= hi
  while (hi > lo) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t p = lo + lane * step;
    const bool le = p < hi && a[p] <= x;
    const int k = __popcll(__ballot(le));  // probes 0 .. k-1 are <= x (the array is sorted)
    if (k == 0) {
      hi = lo;
    } else {
      const int64_t pk = lo + (int64_t)k * step;  // first probe > x, if it exists
      lo += (int64_t)(k - 1) * step + 1;
      if (pk < hi) hi = pk;
    }
  }
  return lo;
}

// four consecutive int32 written with one 16-byte store; the address need only be 4-byte aligned
typedef int32_t int4u __attribute__((ext_vector_type(4), aligned(4)));

// For each k, the number of elements <= x[k] of the sorted LDS array D[0, n).  The K searches run in
// lockstep (the probe offsets halve together), so that their LDS reads are in flight at once instead of
// one dependent chain per search.
template <int K>
__device__ inline void upper_bounds(const int32_t* D, int32_t n, const int32_t (&x)[K], int32_t (&pos)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) pos[k] = 0;
  if (n <= 0) return;
  for (int32_t step = 1 << (31 - __builtin_clz((uint32_t)n)); step > 0; step >>= 1) {
    int32_t v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = D[min(pos[k] + step, n) - 1];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (pos[k] + step <= n && v[k] <= x[k]) pos[k] += step;
  }
}

// Wave-level helpers of k_items_lists (one item per wave, no workgroup barrier).
__device__ inline long long wave_sum(long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// number of lanes below this one whose flag is set
__device__ inline int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  return __popcll(mask & ((1ull << lane) - 1ull));
}
// LDS written by some lanes of this wave becomes visible to every lane of it
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Block-row flags are read in chunks of kRowChunk block columns, kRowLoads byte loads per lane (all in
// flight together): f[u] is block column cbase + u * 64 + lane, 0 past the item's last block column.
constexpr int kRowLoads = 8;
constexpr int kRowChunk = kRowLoads * 64;
__device__ inline void load_row_chunk(const Item& m, int32_t cbase, int lane, uint8_t f[kRowLoads]) {
#pragma unroll
  for (int u = 0; u < kRowLoads; ++u) f[u] = load_in<uint8_t, int32_t>(m.brow, cbase + u * 64 + lane, 0, m.cb1 + 1, 0);
}

// Items per workgroup of k_items_lists (one per wave) and diagonal offsets staged per wave.  When
// the workgroup's items all belong to one head (the usual case: row-block counts are multiples of
// kListWaves), the head's offsets are staged once for the workgroup, in the whole area.
constexpr int kListWaves = 4;
constexpr int kDshWave = 1536;

// Lane 0 stores the four item counters and the scratch slot.
__device__ inline void store_counts_wave(const sa_index& ix, const ItemConsts& kc, const Item& m, long long cnt[4],
                                         uint32_t kind) {
  long long t[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) t[c] = wave_sum(cnt[c]);
  if ((threadIdx.x & 63) == 0) {
    ix.seg_ptr[m.it + 1] = t[0];
    ix.bcol_ptr[m.it + 1] = t[1];
    ix.col_ptr[m.it + 1] = t[2];
    *scratch_slot(ix, kc, m) = ((uint32_t)t[3] & kPairsMask) | (kind << kKindShift);
  }
}

// ---------------------------------------------------------------------------
// Item kinds with no bitmap (blocks only, stripes only, diagonals + verticals).
// One wave per (head, row block), kListWaves items per workgroup; apart from the one
// barrier after a workgroup-wide staging of the head's offsets, the waves never wait for
// each other.  The count pass (fill = 0) classifies the item and, for a
// kKindGeneral item, only records that in its scratch slot.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64 * kListWaves) k_items_lists(sa_pattern_desc d, sa_index ix, int32_t fill,
                                                                 int32_t validate, ItemConsts kc, int32_t n_items) {
  __shared__ int32_t Dsh_all[kListWaves * kDshWave];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t it0 = (int32_t)blockIdx.x * kListWaves, it = it0 + wave;
  const int32_t nbk = ix.n_row_blocks;
  const bool one_head = it0 / nbk == (min(it0 + kListWaves, n_items) - 1) / nbk;  // uniform
  const int32_t dcap = one_head ? kListWaves * kDshWave : kDshWave;  // offsets an item may stage
  // Every wave loads an item (the last one when it has none, so that it can still take part in the
  // staging), and issues with it what the item needs from global memory first: the first chunk of
  // the block row and, in the fill pass, the item's kind and output positions.  They travel
  // together, and with the staging of the head's offsets below.
  const bool has_item = it < n_items;
  const Item m = load_item(d, ix, kc, has_item ? it : n_items - 1);
  const int32_t S = d.S, b0 = m.b0, b1 = m.b1;
  uint8_t f[kRowLoads];  // block-row flags of columns cbase + u * 64 + lane
  if (m.brow != nullptr) load_row_chunk(m, 0, lane, f);
  uint32_t slot = 0;
  int64_t fp_seg = 0, fp_bcol = 0, fp_col = 0, fp_col_end = 0;  // fill pass: the item's first outputs
  if (fill) {
    slot = *scratch_slot(ix, kc, m);
    fp_seg = ix.seg_ptr[m.it];
    fp_bcol = ix.bcol_ptr[m.it];
    fp_col = ix.col_ptr[m.it];
    fp_col_end = ix.col_ptr[m.it + 1];
  }
  const auto uniform_fill_inputs = [&]() {
    slot = uni((int32_t)slot);
    fp_seg = uni64(fp_seg);
    fp_bcol = uni64(fp_bcol);
    fp_col = uni64(fp_col);
    fp_col_end = uni64(fp_col_end);
  };
  __shared__ int32_t n_runs_sh;  // runs of D staged after it (one-head workgroups), or -1
  __shared__ int32_t scan_sh[kListWaves];
  if (one_head) {
    // the head's offsets, once for the workgroup (when they fit; otherwise no item here uses them);
    // every wave's m is an item of this head
    const int32_t nD = m.nD;
    if (nD <= dcap)
      for (int32_t pb = 0; pb < nD; pb += 8 * 64 * kListWaves) {
        int32_t r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          r[u] = load_in<int32_t, int32_t>(m.D, pb + u * 64 * kListWaves + (int32_t)threadIdx.x, 0, nD, 0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int32_t p = pb + u * 64 * kListWaves + (int32_t)threadIdx.x;
          if (p < nD) Dsh_all[p] = r[u];
        }
      }
    __syncthreads();
    // the maximal runs of D, as run_lo at Dsh_all[nD + k] and run_hi at Dsh_all[nD + nruns + k] (when
    // they fit after D): thread t takes a contiguous range of offsets, the run starts before it come
    // from a workgroup scan, and the run ending at an offset is the last one started at or before it
    if (nD > 0 && nD <= dcap) {
      const int32_t per = (nD + 64 * kListWaves - 1) / (64 * kListWaves);
      const int32_t p0 = min(nD, (int32_t)threadIdx.x * per), p1 = min(nD, p0 + per);
      int32_t starts = 0;
      for (int32_t q = p0; q < p1; ++q) starts += (q == 0 || starts_run(Dsh_all[q], Dsh_all[q - 1])) ? 1 : 0;
      int32_t total;
      int32_t k = block_exscan<int32_t>(starts, &total, scan_sh);
      if (nD + 2 * total <= dcap) {
        int32_t* RL = Dsh_all + nD;
        int32_t* RH = Dsh_all + nD + total;
        for (int32_t q = p0; q < p1; ++q) {
          const int32_t r = Dsh_all[q];
          if (q == 0 || starts_run(r, Dsh_all[q - 1])) RL[k++] = r;
          if (q == nD - 1 || starts_run(Dsh_all[q + 1], r)) RH[k - 1] = r;
        }
      }
      if (threadIdx.x == 0) n_runs_sh = nD + 2 * total <= dcap ? total : -1;
    } else if (threadIdx.x == 0) {
      n_runs_sh = -1;
    }
    __syncthreads();
  }
  if (!has_item) return;  // the whole wave leaves; nothing below waits for other waves
  int32_t* Dsh = one_head ? Dsh_all : Dsh_all + wave * kDshWave;

  uint32_t kind;
  long long blk_cols = 0, blk_pairs = 0;  // the block-mask columns' counts, used if the item is block-only
  if (!fill) {
    int any = 0;
    if (m.brow != nullptr) {
      const int32_t bs = kc.bs;
      for (int32_t cbase = 0; cbase <= m.cb1; cbase += kRowChunk) {
        if (cbase > 0) load_row_chunk(m, cbase, lane, f);
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
          if (f[u]) {
            const int32_t c0 = (cbase + u * 64 + lane) * bs, c1 = min(b1, c0 + bs - 1);
            any = 1;
            blk_cols += c1 - c0 + 1;
            blk_pairs += column_pairs(c0, c1, b0, b1);
          }
        }
      }
    }
    const bool has_blk = __ballot(any != 0) != 0ull;
    const bool has_vert = m.vp1 > m.vp0, has_str = m.sp1 > m.sp0, has_diag = m.nD > 0;
    if (has_blk && !has_diag && !has_vert && !has_str) kind = kKindBlocks;
    else if (has_str && !has_blk && !has_diag && !has_vert) kind = kKindStripes;
    else if (!has_blk && !has_str && m.nD <= dcap) kind = kKindLists;
    else kind = kKindGeneral;
    if (kind == kKindGeneral) {
      if (lane == 0) *scratch_slot(ix, kc, m) = kKindGeneral << kKindShift;
      return;
    }
  } else {
    uniform_fill_inputs();
    kind = slot >> kKindShift;
    if (kind == kKindGeneral) return;
  }

  long long cnt[4] = {0, 0, 0, 0};  // segments, in-segment columns, gathered columns, retained pairs
  bool bad = false, overflow = false;

  if (kind == kKindBlocks) {
    const int32_t bs = kc.bs;
    if (!fill) {
      cnt[2] = blk_cols;
      cnt[3] = blk_pairs;
      store_counts_wave(ix, kc, m, cnt, kind);
      return;
    }
    // fill: every set block but the last is full, so set block k of the row (in order) starts at
    // output k * bs.
    const int64_t base = fp_col;
    const int64_t cap = ix.capacity.n_cols;
    int64_t done = 0;  // set blocks before the current chunk of block columns
    if (bs == 64) {
      // The set block columns of each chunk of kRowChunk are compacted into this wave's LDS area (in
      // order: rank from the ballots), then written four blocks per store instruction: lanes
      // 16q .. 16q + 15 write block t + q, four columns (16 bytes) each.  Only a block-only item takes
      // this path, and its head has no diagonal offsets, so no wave of the workgroup uses the staging
      // area for them.
      int32_t* sel = Dsh_all + wave * kDshWave;
      const uint64_t below = (1ull << lane) - 1ull;
      for (int32_t cbase = 0; cbase <= m.cb1; cbase += kRowChunk) {
        if (cbase > 0) load_row_chunk(m, cbase, lane, f);
        int32_t n = 0;
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
          const uint64_t set0 = __ballot(f[u] != 0);
          if (f[u]) sel[n + __popcll(set0 & below)] = cbase + u * 64 + lane;
          n += __popcll(set0);
        }
        wave_lds_sync();
        const int q = lane >> 4, e4 = 4 * (lane & 15);
        for (int32_t t = 0; t < n; t += 4) {
          const int32_t tq = t + q;
          if (tq < n) {
            const int32_t c0 = sel[tq] * 64, c1 = min(b1, c0 + 63), c = c0 + e4;
            const int64_t pos = base + (done + tq) * 64 + e4;
            if (c + 3 <= c1 && pos + 3 < cap) {
              *reinterpret_cast<int4u*>(ix.col_idx + pos) = int4u{c, c + 1, c + 2, c + 3};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (c + e <= c1) {
                  if (pos + e < cap) ix.col_idx[pos + e] = c + e; else overflow = true;
                }
              }
            }
          }
        }
        done += n;
        wave_lds_sync();  // every lane has read `sel` before the next chunk overwrites it
      }
    } else {
      for (int32_t cbase = 0; cbase <= m.cb1; cbase += kRowChunk) {
        if (cbase > 0) load_row_chunk(m, cbase, lane, f);
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
          const uint64_t set0 = __ballot(f[u] != 0);
          uint64_t set = set0;
          while (set) {
            const int j = __ffsll((unsigned long long)set) - 1;
            const int64_t k = done + __popcll(set0 & ((1ull << j) - 1ull));  // set blocks before this one
            set &= set - 1;
            const int32_t c0 = (cbase + u * 64 + j) * bs, c1 = min(b1, c0 + bs - 1);
            for (int32_t c = c0 + lane; c <= c1; c += 64) {
              const int64_t pos = base + k * bs + (c - c0);
              if (pos < cap) ix.col_idx[pos] = c; else overflow = true;
            }
          }
          done += __popcll(set0);
        }
      }
    }
  } else if (kind == kKindStripes) {
    if (!fill && !validate) {
      // sorted list: entries below b0 each give every row; the few in [b0, b1] are summed one by one
      const int64_t len = m.sp1 - m.sp0;
      const int64_t n_le = wave_upper_bound(d.stripe_col + m.sp0, len, b1);
      const int64_t n_lt = wave_upper_bound(d.stripe_col + m.sp0, n_le, b0 - 1);
      if (lane == 0) {
        cnt[2] = n_le;
        cnt[3] = n_lt * (long long)(b1 - b0 + 1);
      }
      for (int64_t q = n_lt + lane; q < n_le; q += 64) {
        const int32_t c = d.stripe_col[m.sp0 + q];
        cnt[3] += b1 - max(c, b0) + 1;
      }
      store_counts_wave(ix, kc, m, cnt, kind);
      return;
    }
    if (!fill) {
      for (int64_t pb = m.sp0; pb < m.sp1; pb += 8 * 64) {
        int32_t c[8], prev[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t p = pb + u * 64 + lane;
          c[u] = load_in<int32_t, int64_t>(d.stripe_col, p, m.sp0, m.sp1, -1);
          prev[u] = load_in<int32_t, int64_t>(d.stripe_col, p - 1, m.sp0, m.sp1, -1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t p = pb + u * 64 + lane;
          if (p < m.sp1 && (c[u] < 0 || c[u] >= S || (p > m.sp0 && prev[u] >= c[u]))) bad = true;
          if (c[u] >= 0 && c[u] <= b1) {
            cnt[2] += 1;
            cnt[3] += b1 - max(c[u], b0) + 1;
          }
        }
      }
      if (bad) atomicOr(ix.status, SA_STATUS_DESC_INVALID);
      store_counts_wave(ix, kc, m, cnt, kind);
      return;
    }
    // fill: the columns <= b1 of a sorted list are its first n entries
    const int64_t base = fp_col, n = fp_col_end - base;
    const int64_t cap = ix.capacity.n_cols;
    for (int64_t qb = 0; qb < n; qb += 8 * 64) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = qb + u * 64 + lane;
        c[u] = load_in<int32_t, int64_t>(d.stripe_col + m.sp0, q, 0, n, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = qb + u * 64 + lane;
        if (q < n) {
          int32_t col = c[u];
          if (col < 0 || col > b1) {  // only an unsorted list gets here; keep every column in range
            bad = true;
            col = min(max(col, 0), b1);
          }
          if (base + q < cap) ix.col_idx[base + q] = col; else overflow = true;
        }
      }
    }
  } else {  // kKindLists
    const int32_t nD = m.nD;
    for (int32_t pb = 0; !one_head && pb < nD; pb += 8 * 64) {  // staged per wave
      int32_t r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int32_t p = pb + u * 64 + lane;
        r[u] = load_in<int32_t, int32_t>(m.D, p, 0, nD, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int32_t p = pb + u * 64 + lane;
        if (p < nD) Dsh[p] = r[u];
      }
    }
    wave_lds_sync();
    // A run [lo, hi] of D (lo <= b1) touches key columns I = [max(0, b0 - hi), b1 - lo] (clipped to
    // [0, b1]); runs in descending offset order give intervals in ascending column order, and U's
    // segments are the merged intervals.  The run with the next larger offsets starts at index q + 1
    // (q: this run's last index); the one with the next smaller offsets ends at index p - 1.
    auto run_of = [&](int32_t p, int32_t& lo, int32_t& hi, int32_t& q) {
      lo = Dsh[p];
      int32_t qa = p, qb = nD - 1;
      while (qa < qb) {
        const int32_t mid = (qa + qb + 1) >> 1;
        if (Dsh[mid] - mid == lo - p) qa = mid;
        else qb = mid - 1;
      }
      q = qa;
      hi = Dsh[qa];
    };
    auto is_run_start = [&](int32_t p) { return p == 0 || starts_run(Dsh[p], Dsh[p - 1]); };
    auto seg_flags = [&](int32_t p, bool& st, bool& en, int32_t& s0, int32_t& s1) {
      st = en = false;
      if (p < 0 || p >= nD || !is_run_start(p)) return;
      int32_t lo, hi, q;
      run_of(p, lo, hi, q);
      if (lo > b1) return;
      s0 = max(0, b0 - hi);
      s1 = min(b1, b1 - lo);
      st = !(q + 1 < nD && Dsh[q + 1] <= b1 && s0 <= min(b1, b1 - Dsh[q + 1]) + 1);
      en = !(p > 0 && max(0, b0 - Dsh[p - 1]) <= s1 + 1);
    };

    // with the runs staged: the same flags from run k and its neighbours, no search
    const int32_t nr = one_head ? n_runs_sh : -1;
    const int32_t* RL = Dsh + nD;
    const int32_t* RH = Dsh + nD + max(nr, 0);
    auto run_flags = [&](int32_t k, bool& st, bool& en, int32_t& s0, int32_t& s1) {
      st = en = false;
      if (k < 0 || k >= nr) return;
      const int32_t lo = RL[k], hi = RH[k];
      if (lo > b1) return;
      s0 = max(0, b0 - hi);
      s1 = min(b1, b1 - lo);
      st = !(k + 1 < nr && RL[k + 1] <= b1 && s0 <= min(b1, b1 - RL[k + 1]) + 1);
      en = !(k > 0 && max(0, b0 - RH[k - 1]) <= s1 + 1);
    };

    if (!fill) {
      if (nr >= 0) {
        for (int32_t k = lane; k < nr; k += 64) {
          bool st, en;
          int32_t s0, s1;
          run_flags(k, st, en, s0, s1);
          cnt[0] += st ? 1 : 0;
        }
      } else {
      // segments start at runs of D: four offsets per lane and step, their reads issued together
      for (int32_t pb = 0; pb < nD; pb += 4 * 64) {
        bool start[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int32_t p = min(pb + k * 64 + lane, nD - 1);
          start[k] = p == 0 || starts_run(Dsh[p], Dsh[max(p - 1, 0)]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int32_t p = pb + k * 64 + lane;
          if (p < nD && start[k]) {
            bool st, en;
            int32_t s0, s1;
            seg_flags(p, st, en, s0, s1);
            cnt[0] += st ? 1 : 0;
          }
        }
      }
      }
      // verticals: the offsets of D in [a - c, b1 - c] (a = max(b0, c)) are the rows of the block that
      // reach c along a diagonal
      for (int32_t pb = m.vp0; pb < m.vp1; pb += 8 * 64) {
        int32_t c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int32_t p = pb + u * 64 + lane;
          c[u] = load_in<int32_t, int32_t>(d.vert_col, p, m.vp0, m.vp1, -1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (c[u] < 0 || c[u] > b1) continue;
          const int32_t a = max(b0, c[u]);
          const int32_t dc = upper_bound_i32(Dsh, nD, b1 - c[u]) - upper_bound_i32(Dsh, nD, a - c[u] - 1);
          if (dc > 0) {
            cnt[1] += 1;
            cnt[3] += (b1 - a + 1) - dc;
          } else {
            cnt[2] += 1;
            cnt[3] += b1 - a + 1;
          }
        }
      }
      // diagonal pairs of each row: offsets r in D_h with r <= i (BM <= 128: two rows per lane)
      if (nD > 0) {
        int32_t x[2] = {b0 + lane, b0 + 64 + lane}, ub[2];
        upper_bounds<2>(Dsh, nD, x, ub);
        if (x[0] <= b1) cnt[3] += ub[0];
        if (x[1] <= b1) cnt[3] += ub[1];
      }
      store_counts_wave(ix, kc, m, cnt, kind);
      return;
    }
    // fill: segments in ascending column order = runs in descending offset order
    int64_t bs_lo = fp_seg, bs_hi = bs_lo;
    for (int32_t kb = 0; nr >= 0 && kb < nr; kb += 64) {
      bool st, en;
      int32_t s0 = 0, s1 = 0;
      run_flags(nr - 1 - (kb + lane), st, en, s0, s1);
      const uint64_t mst = __ballot(st), men = __ballot(en);
      if (st) {
        const int64_t pos = bs_lo + lanes_below(mst);
        if (pos < ix.capacity.n_segs) ix.seg_lo[pos] = s0; else overflow = true;
      }
      if (en) {
        const int64_t pos = bs_hi + lanes_below(men);
        if (pos < ix.capacity.n_segs) ix.seg_hi[pos] = s1; else overflow = true;
      }
      bs_lo += __popcll(mst);
      bs_hi += __popcll(men);
    }
    for (int32_t cb4 = 0; nr < 0 && cb4 < nD; cb4 += 4 * 64) {
      // which of the next 4 x 64 offsets start a run (reads issued together); steps with none are skipped
      bool start[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int32_t p = nD - 1 - (cb4 + k * 64 + lane), pc = max(p, 0);
        start[k] = p >= 0 && (pc == 0 || starts_run(Dsh[pc], Dsh[max(pc - 1, 0)]));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (__ballot(start[k]) == 0ull) continue;
        const int32_t p = nD - 1 - (cb4 + k * 64 + lane);
        bool st = false, en = false;
        int32_t s0 = 0, s1 = 0;
        if (start[k]) seg_flags(p, st, en, s0, s1);
        const uint64_t mst = __ballot(st), men = __ballot(en);
        if (st) {
          const int64_t pos = bs_lo + lanes_below(mst);
          if (pos < ix.capacity.n_segs) ix.seg_lo[pos] = s0; else overflow = true;
        }
        if (en) {
          const int64_t pos = bs_hi + lanes_below(men);
          if (pos < ix.capacity.n_segs) ix.seg_hi[pos] = s1; else overflow = true;
        }
        bs_lo += __popcll(mst);
        bs_hi += __popcll(men);
      }
    }
    // verticals in list order, split into in-segment and gathered columns
    int64_t b_in = fp_bcol, b_out = fp_col;
    for (int32_t pb = m.vp0; pb < m.vp1; pb += 64) {
      const int32_t p = pb + lane;
      const int32_t c = p < m.vp1 ? d.vert_col[p] : -1;
      bool in = false, out = false;
      const bool ok = c >= 0 && c <= b1;
      int32_t x[2] = {ok ? b1 - c : -1, ok ? max(b0, c) - c - 1 : -1}, ub[2];
      upper_bounds<2>(Dsh, nD, x, ub);
      if (ok) {
        if (ub[0] > ub[1]) in = true;
        else out = true;
      }
      const uint64_t min_ = __ballot(in), mout = __ballot(out);
      if (in) {
        const int64_t pos = b_in + lanes_below(min_);
        if (pos < ix.capacity.n_bcols) ix.bcol_idx[pos] = c; else overflow = true;
      }
      if (out) {
        const int64_t pos = b_out + lanes_below(mout);
        if (pos < ix.capacity.n_cols) ix.col_idx[pos] = c; else overflow = true;
      }
      b_in += __popcll(min_);
      b_out += __popcll(mout);
    }
  }
  if (bad) atomicOr(ix.status, SA_STATUS_DESC_INVALID);
  if (overflow) atomicOr(ix.status, SA_STATUS_OVERFLOW);
}

// Gathered-column slots per thread and round of the bitmap fill: thread t expands slots
// [kSlots t, kSlots t + kSlots) of the round into an LDS stage, then the workgroup stores the
// round's kSlots * kThreads slots coalesced.
constexpr int kSlots = 8;
static_assert(kSlots * kThreads <= kDsh, "the fill stage lives in the diagonal staging area");

// ---------------------------------------------------------------------------
// Bitmap path (items of kind kKindGeneral; the others return at once): build X
// and U bitmaps over key columns [0, b1], then count (fill = 0) or write (fill = 1)
// segments, in-segment columns and gathered columns.
// STAGED: the head's diagonal offsets are in LDS (searched with LDS reads).
// ---------------------------------------------------------------------------
template <bool STAGED>
__device__ inline void items_body(const sa_pattern_desc& d, const sa_index& ix, int32_t fill, int32_t validate,
                                  const ItemConsts& kc, const Item& m, const int32_t* Dq, uint32_t* X, uint32_t* U,
                                  int32_t* scan_sh, long long* red_sh, int32_t* off_sh, int32_t* stage) {
  const int tid = threadIdx.x;
  const int32_t S = d.S, b0 = m.b0, b1 = m.b1, nw = m.nw, nD = m.nD;
  // --- verticals and stripe columns into X (eight loads in flight per thread)
  for (int32_t pb = m.vp0; pb < m.vp1; pb += 8 * kThreads) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int32_t p = pb + u * kThreads + tid;
      c[u] = load_in<int32_t, int32_t>(d.vert_col, p, m.vp0, m.vp1, -1);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c[u] >= 0 && c[u] <= b1) atomicOr(&X[c[u] >> 5], 1u << (c[u] & 31));
  }
  if (m.sp1 > m.sp0) {
    bool bad = false;
    for (int64_t pb = m.sp0; pb < m.sp1; pb += 8 * kThreads) {
      int32_t c[8], prev[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t p = pb + u * kThreads + tid;
        c[u] = load_in<int32_t, int64_t>(d.stripe_col, p, m.sp0, m.sp1, -1);
        prev[u] = validate ? load_in<int32_t, int64_t>(d.stripe_col, p - 1, m.sp0, m.sp1, -1) : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t p = pb + u * kThreads + tid;
        if (validate && p < m.sp1 && (c[u] < 0 || c[u] >= S || (p > m.sp0 && prev[u] >= c[u]))) bad = true;
        if (c[u] >= 0 && c[u] <= b1) atomicOr(&X[c[u] >> 5], 1u << (c[u] & 31));
      }
    }
    if (bad && !fill) atomicOr(ix.status, SA_STATUS_DESC_INVALID);
  }
  // --- U: columns i - r for i in [b0, b1] and r in a run [lo, hi] of D_h: [b0 - hi, b1 - lo], clipped
  // to [0, b1].  Staged offsets: a thread that holds the first offset of a run finds the run's end by
  // binary search (D[q] - q is non-decreasing and constant exactly along a run).  Offsets in global
  // memory: each offset r <= b1 sets its own columns [b0 - r, b1 - r] (the union is the same), eight
  // loads in flight per thread and no search.
  if constexpr (!STAGED) {
    for (int32_t pb = 0; pb < nD; pb += 8 * kThreads) {
      int32_t r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = load_in<int32_t, int32_t>(Dq, pb + u * kThreads + tid, 0, nD, INT32_MAX);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r[u] > b1) continue;
        const int32_t a = max(0, b0 - r[u]), e = b1 - r[u];
        for (int32_t w = a >> 5; w <= (e >> 5); ++w) {
          const int32_t ba = max(a, w * 32) - w * 32, be = min(e, w * 32 + 31) - w * 32;
          atomicOr(&U[w], bit_range(ba, be));
        }
      }
    }
  }
  for (int32_t p = tid; STAGED && p < nD; p += kThreads) {
    const int32_t lo = Dq[p];
    if (p > 0 && !starts_run(lo, Dq[p - 1])) continue;  // not the first offset of a run
    if (lo > b1) continue;
    int32_t qa = p, qb = nD - 1;
    while (qa < qb) {
      const int32_t mid = (qa + qb + 1) >> 1;
      if (Dq[mid] - mid == lo - p) qa = mid;
      else qb = mid - 1;
    }
    const int32_t hi = Dq[qa];
    const int32_t a = max(0, b0 - hi), e = min(b1, b1 - lo);
    for (int32_t w = a >> 5; a <= e && w <= (e >> 5); ++w) {
      const int32_t ba = max(a, w * 32) - w * 32, be = min(e, w * 32 + 31) - w * 32;
      atomicOr(&U[w], bit_range(ba, be));
    }
  }
  __syncthreads();

  if (!fill) {
    long long cnt[4] = {0, 0, 0, 0};  // segments, in-segment columns, gathered columns, retained pairs
    for (int32_t w = tid; w < nw; w += kThreads) {
      const uint32_t u = U[w], x = X[w];
      const uint32_t prev_msb = (w > 0) ? (U[w - 1] >> 31) : 0u;
      cnt[0] += __popc(u & ~((u << 1) | prev_msb));
      uint32_t in = x & u, out = x & ~u;
      cnt[1] += __popc(in);
      cnt[2] += __popc(out);
      // gathered columns: rows max(j, b0) .. b1, all retained
      if (w * 32 + 31 < b0) {
        cnt[3] += (long long)__popc(out) * (long long)(b1 - b0 + 1);
      } else {
        while (out) {
          int bit = __ffs(out) - 1;
          out &= out - 1;
          int32_t j = w * 32 + bit;
          cnt[3] += b1 - max(j, b0) + 1;
        }
      }
      // in-segment columns of X: every causal row minus the rows whose offset is a diagonal (with the
      // offsets in global memory, those rows are taken off per offset below)
      while (in) {
        int bit = __ffs(in) - 1;
        in &= in - 1;
        int32_t j = w * 32 + bit;
        int32_t a = max(j, b0);
        const int32_t dcount = STAGED ? upper_bound_i32(Dq, nD, b1 - j) - upper_bound_i32(Dq, nD, a - j - 1) : 0;
        cnt[3] += (b1 - a + 1) - dcount;
      }
    }
    if constexpr (STAGED) {
      // diagonal pairs of each row: offsets r in D_h with r <= i
      if (nD > 0)
        for (int32_t i = b0 + tid; i <= b1; i += kThreads) cnt[3] += upper_bound_i32(Dq, nD, i);
    } else {
      // per offset r <= b1: its rows max(r, b0) .. b1 (diagonal pairs), less the in-segment columns j
      // in [b0 - r, b1 - r], whose pair (j + r, j) was counted with the column above
      for (int32_t pb = 0; pb < nD; pb += 8 * kThreads) {
        int32_t r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = load_in<int32_t, int32_t>(Dq, pb + u * kThreads + tid, 0, nD, INT32_MAX);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (r[u] > b1) continue;
          cnt[3] += b1 - max(r[u], b0) + 1;
          const int32_t a = max(0, b0 - r[u]), e = b1 - r[u];
          for (int32_t w = a >> 5; w <= (e >> 5); ++w) {
            const int32_t ba = max(a, w * 32) - w * 32, be = min(e, w * 32 + 31) - w * 32;
            cnt[3] -= __popc(X[w] & U[w] & bit_range(ba, be));
          }
        }
      }
    }
    store_counts(ix, kc, m, cnt, kKindGeneral, red_sh);
    return;
  }

  // --- fill: four consecutive words per thread per chunk, block scan for write positions.  Segment
  // ends and in-segment columns are few and each thread writes its own.  Gathered columns are many:
  // thread t expands the kSlots consecutive output slots starting at slot kSlots * t of the round (one
  // search over the per-thread offsets, then a walk along the chunk's words) into the LDS stage, which
  // the workgroup then stores with consecutive threads on consecutive slots.  The stage reuses the
  // diagonal staging area: the fill reads no diagonal offset after U is built.
  int64_t base_rise = ix.seg_ptr[m.it], base_fall = base_rise, base_in = ix.bcol_ptr[m.it],
          base_out = ix.col_ptr[m.it];
  bool overflow = false;
  const int64_t cap_out = ix.capacity.n_cols;
  for (int32_t w0 = 0; w0 < nw; w0 += 4 * kThreads) {
    const int32_t wt = w0 + 4 * tid;
    const int32_t wend = min(nw, w0 + 4 * kThreads);  // words of this chunk: [w0, wend)
    uint32_t rise[4], fall[4], in[4];
    int32_t v[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t w = wt + u;
      rise[u] = fall[u] = in[u] = 0;
      if (w < nw) {
        const uint32_t uu = U[w], x = X[w];
        const uint32_t prev_msb = (w > 0) ? (U[w - 1] >> 31) : 0u;
        const uint32_t next_lsb = (w + 1 < nw) ? (U[w + 1] & 1u) : 0u;
        rise[u] = uu & ~((uu << 1) | prev_msb);
        fall[u] = uu & ~((uu >> 1) | (next_lsb << 31));
        in[u] = x & uu;
        v[3] += __popc(x & ~uu);
      }
      v[0] += __popc(rise[u]);
      v[1] += __popc(fall[u]);
      v[2] += __popc(in[u]);
    }
    int32_t tot[4];
    block_scan4(v, tot, scan_sh);
    off_sh[tid] = v[3];
    int64_t pr = base_rise + v[0], pf = base_fall + v[1], pi = base_in + v[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t wcol = (wt + u) * 32;
      uint32_t mk = rise[u];
      while (mk) {
        int bit = __ffs(mk) - 1;
        mk &= mk - 1;
        if (pr < ix.capacity.n_segs) ix.seg_lo[pr] = wcol + bit; else overflow = true;
        ++pr;
      }
      mk = fall[u];
      while (mk) {
        int bit = __ffs(mk) - 1;
        mk &= mk - 1;
        if (pf < ix.capacity.n_segs) ix.seg_hi[pf] = wcol + bit; else overflow = true;
        ++pf;
      }
      mk = in[u];
      while (mk) {
        int bit = __ffs(mk) - 1;
        mk &= mk - 1;
        if (pi < ix.capacity.n_bcols) ix.bcol_idx[pi] = wcol + bit; else overflow = true;
        ++pi;
      }
    }
    __syncthreads();  // off_sh complete
    for (int32_t qb = 0; qb < tot[3]; qb += kSlots * kThreads) {
      const int32_t q0 = qb + kSlots * tid;
      if (q0 < tot[3]) {
        // owner of slot q0: the last thread t with off_sh[t] <= q0
        int32_t lo = 0, hi = kThreads - 1;
        while (lo < hi) {
          const int32_t mid = (lo + hi + 1) >> 1;
          if (off_sh[mid] <= q0) lo = mid;
          else hi = mid - 1;
        }
        int32_t k = q0 - off_sh[lo];
        int32_t w = w0 + 4 * lo;
        uint32_t cur = X[w] & ~U[w];
        while (k >= __popc(cur)) {  // the slot lies in one of the owner's four words
          k -= __popc(cur);
          ++w;
          cur = (w < wend) ? (X[w] & ~U[w]) : 0u;
        }
        for (; k > 0; --k) cur &= cur - 1;
        const int32_t n = min(kSlots, tot[3] - q0);
#pragma unroll
        for (int e = 0; e < kSlots; ++e) {
          if (e < n) {
            while (cur == 0 && w + 1 < wend) {
              ++w;
              cur = X[w] & ~U[w];
            }
            stage[kSlots * tid + e] = w * 32 + __ffs(cur) - 1;
            cur &= cur - 1;
          }
        }
      }
      __syncthreads();  // the round's slots are in stage, in slot order
      const int64_t pos = base_out + qb;
#pragma unroll
      for (int e = 0; e < kSlots; ++e) {
        const int32_t sidx = e * kThreads + tid;
        if (qb + sidx < tot[3]) {
          if (pos + sidx < cap_out) ix.col_idx[pos + sidx] = stage[sidx]; else overflow = true;
        }
      }
      __syncthreads();  // stage reused by the next round
    }
    __syncthreads();  // off_sh reused by the next chunk
    base_rise += tot[0];
    base_fall += tot[1];
    base_in += tot[2];
    base_out += tot[3];
  }
  if (overflow) atomicOr(ix.status, SA_STATUS_OVERFLOW);
}

// Items per workgroup of k_items: the kinds of kGenBatch items (strided by the grid) are read at
// once, and the workgroup builds the general ones among them one after another.
constexpr int kGenBatch = 16;

__global__ void __launch_bounds__(kThreads) k_items(sa_pattern_desc d, sa_index ix, int32_t fill, int32_t validate,
                                                    ItemConsts kc, int32_t n_items) {
  extern __shared__ uint32_t lds[];
  __shared__ int32_t scan_sh[kWaves * 4];
  __shared__ long long red_sh[kWaves * 4];
  __shared__ int32_t off_sh[kThreads];

  const int tid = threadIdx.x;
  uint32_t* X = lds;
  uint32_t* U = lds + kc.nwords;
  int32_t* Dsh = reinterpret_cast<int32_t*>(lds + 2 * kc.nwords);
  const int32_t nbatch = (int32_t)gridDim.x;
  bool general = false;
  if (tid < kGenBatch) {
    const int32_t it = (int32_t)blockIdx.x + tid * nbatch;
    if (it < n_items) {
      const int32_t h = it / ix.n_row_blocks, rb = it - h * ix.n_row_blocks;
      general = (ix.dbits[(int64_t)h * kc.nwords + rb] >> kKindShift) == kKindGeneral;
    }
  }
  uint64_t todo = __ballot(general);  // bits of wave 0 (tid < kGenBatch <= 64)
  __shared__ uint64_t todo_sh;
  if (tid == 0) todo_sh = todo;
  __syncthreads();
  todo = todo_sh;

  while (todo) {
    const int j = __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const Item m = load_item(d, ix, kc, (int32_t)blockIdx.x + j * nbatch);
    const int32_t b1 = m.b1, nw = m.nw, nD = m.nD;
    const bool staged = nD <= kc.dcap;

    // --- X from the block row, U cleared, D staged in LDS
    const int32_t blk_end = (kc.wpb_shift >= 0 ? ((nw - 1) >> kc.wpb_shift) : (nw - 1) / kc.wpb) + 1;
    for (int32_t wb = 0; wb < nw; wb += 4 * kThreads) {
      uint32_t x[4] = {0u, 0u, 0u, 0u};
      if (m.brow != nullptr) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int32_t w = wb + u * kThreads + tid;
          const int32_t blk = kc.wpb_shift >= 0 ? (w >> kc.wpb_shift) : w / kc.wpb;
          x[u] = load_in<uint8_t, int32_t>(m.brow, blk, 0, blk_end, 0) ? 0xffffffffu : 0u;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int32_t w = wb + u * kThreads + tid;
        if (w < nw) {
          X[w] = (w == nw - 1) ? (x[u] & bit_range(0, b1 & 31)) : x[u];
          U[w] = 0;
        }
      }
    }
    if (staged) {
      for (int32_t pb = 0; pb < nD; pb += 8 * kThreads) {
        int32_t r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int32_t p = pb + u * kThreads + tid;
          r[u] = load_in<int32_t, int32_t>(m.D, p, 0, nD, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int32_t p = pb + u * kThreads + tid;
          if (p < nD) Dsh[p] = r[u];
        }
      }
    }
    __syncthreads();
    if (staged)
      items_body<true>(d, ix, fill, validate, kc, m, Dsh, X, U, scan_sh, red_sh, off_sh, Dsh);
    else
      items_body<false>(d, ix, fill, validate, kc, m, m.D, X, U, scan_sh, red_sh, off_sh, Dsh);
    __syncthreads();  // LDS reused by the next item
  }
}

// ---------------------------------------------------------------------------
// Scans of the item pointer arrays: entries 1..n hold per-item counts (entry 0
// becomes 0); afterwards ptr[it] is the first element of item it.  Three passes
// over chunks of kScanChunk entries, in place:
//   local   each chunk scanned on its own (its last entry is then the chunk total)
//   offset  every entry but a chunk's last gets the sum of the earlier chunk totals
//   fix     one workgroup adds the same sums to the chunks' last entries, scans the
//           per-head run counts into run_ptr and folds invalid-head marks into status
// ---------------------------------------------------------------------------
__device__ inline int64_t* pick(int64_t* a0, int64_t* a1, int64_t* a2, int which) {
  return which == 0 ? a0 : (which == 1 ? a1 : a2);
}

__global__ void __launch_bounds__(kThreads) k_scan_local(int64_t* a0, int64_t* a1, int64_t* a2, int64_t n) {
  __shared__ long long sh[kWaves];
  int64_t* a = pick(a0, a1, a2, blockIdx.y);
  const int64_t c = blockIdx.x;
  const int64_t end = min(n, (c + 1) * kScanChunk);
  const int64_t base = 1 + c * kScanChunk + (int64_t)threadIdx.x * kScanPer;
  long long v[kScanPer], s = 0;
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) v[u] = load_in<int64_t, int64_t>(a, base + u, 1, end + 1, 0);
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) s += v[u];
  long long tot;
  long long run = block_exscan<long long>(s, &tot, sh);
#pragma unroll
  for (int u = 0; u < kScanPer; ++u) {
    run += v[u];
    if (base + u <= end) a[base + u] = run;
  }
}

__global__ void __launch_bounds__(kThreads) k_scan_offset(int64_t* a0, int64_t* a1, int64_t* a2, int64_t n) {
  __shared__ long long sh[kWaves];
  const int64_t c = blockIdx.x;
  if (c == 0) return;
  int64_t* a = pick(a0, a1, a2, blockIdx.y);
  long long part = 0;
  for (int64_t cc = threadIdx.x; cc < c; cc += kThreads) part += a[(cc + 1) * kScanChunk];  // full chunks
  const long long off = block_sum<long long>(part, sh);
  const int64_t end = min(n, (c + 1) * kScanChunk);
  const int64_t base = 1 + c * kScanChunk + (int64_t)threadIdx.x * kScanPer;
#pragma unroll
  for (int u = 0; u < kScanPer; ++u)
    if (base + u < end) a[base + u] += off;
}

__global__ void __launch_bounds__(kThreads) k_scan_fix(int64_t* a0, int64_t* a1, int64_t* a2, int64_t n,
                                                       int32_t* run_ptr, int32_t n_heads, int32_t* status) {
  __shared__ long long sh[kWaves];
  __shared__ int32_t sh32[kWaves];
  const int tid = threadIdx.x;
  const int64_t C = (n + kScanChunk - 1) / kScanChunk;
  for (int which = 0; which < 3; ++which) {
    int64_t* a = pick(a0, a1, a2, which);
    long long carry = 0;
    for (int64_t cb = 0; cb < C; cb += kThreads) {
      const int64_t c = cb + tid;
      const int64_t e = min(n, (c + 1) * kScanChunk);
      const long long t = c < C ? a[e] : 0;
      long long tot;
      const long long ex = block_exscan<long long>(t, &tot, sh);
      if (c < C) a[e] = carry + ex + t;
      carry += tot;
    }
    if (tid == 0) a[0] = 0;
  }
  int32_t carry = 0, bad = 0;
  for (int32_t hb = 0; hb < n_heads; hb += kThreads) {
    const int32_t hh = hb + tid;
    int32_t v = load_in<int32_t, int32_t>(run_ptr, hh + 1, 1, n_heads + 1, 0);
    bad |= v & kBadHead;
    v &= ~kBadHead;
    int32_t tot;
    const int32_t ex = block_exscan<int32_t>(v, &tot, sh32);
    if (hh < n_heads) run_ptr[hh + 1] = carry + ex + v;
    carry += tot;
  }
  bad = block_sum<int32_t>(bad ? 1 : 0, sh32);
  if (tid == 0 && bad) atomicOr(status, SA_STATUS_DESC_INVALID);
}

// ---------------------------------------------------------------------------
// Per head, after the fill: pair_count[h] from the items' scratch slots in dbits
// row h, then the D bitmap over that row (built in LDS), then the maximal runs of
// D at run_ptr[h] (run_ptr already scanned).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) k_heads_fill(sa_pattern_desc d, sa_index ix, int32_t nwords) {
  extern __shared__ uint32_t bits[];  // [nwords]
  __shared__ int32_t sh[kWaves];
  __shared__ long long shl[kWaves];
  const int tid = threadIdx.x;
  const int32_t h = blockIdx.x, S = d.S, nb = ix.n_row_blocks;
  uint32_t* row = ix.dbits + (int64_t)h * nwords;
  long long pairs = 0;
  for (int32_t rb = tid; rb < nb; rb += kThreads) pairs += row[rb] & kPairsMask;
  for (int32_t w = tid; w < nwords; w += kThreads) bits[w] = 0;
  pairs = block_sum<long long>(pairs, shl);  // its barriers: every slot read, bitmap cleared
  if (tid == 0) ix.pair_count[h] = pairs;

  const int32_t p0 = d.diag_ptr[h], p1 = d.diag_ptr[h + 1];
  for (int32_t p = p0 + tid; p < p1; p += kThreads) {
    const int32_t r = d.diag_off[p];
    if (r >= 0 && r < S) atomicOr(&bits[r >> 5], 1u << (r & 31));
  }
  __syncthreads();
  for (int32_t w = tid; w < nwords; w += kThreads) row[w] = bits[w];

  int64_t base = ix.run_ptr[h];
  bool overflow = false;
  for (int32_t pb = p0; pb < p1; pb += kThreads) {
    const int32_t p = pb + tid;
    const bool in = p < p1;
    int32_t r = 0, prev = 0, next = 0;
    if (in) {
      r = d.diag_off[p];
      if (p > p0) prev = d.diag_off[p - 1];
      if (p + 1 < p1) next = d.diag_off[p + 1];
    }
    const bool st = in && (p == p0 || starts_run(r, prev));
    const bool en = in && (p + 1 == p1 || starts_run(next, r));
    int32_t tot;
    const int32_t ex = block_exscan<int32_t>(st ? 1 : 0, &tot, sh);
    const int64_t idx = base + ex + (st ? 1 : 0) - 1;  // the run that holds offset p
    if (st) {
      if (idx < ix.capacity.n_runs) ix.run_lo[idx] = r; else overflow = true;
    }
    if (en) {
      if (idx >= 0 && idx < ix.capacity.n_runs) ix.run_hi[idx] = r; else overflow = true;
    }
    base += tot;
  }
  if (overflow) atomicOr(ix.status, SA_STATUS_OVERFLOW);
}

}  // namespace

hipError_t launch_index_heads(const sa_pattern_desc& d, const sa_index& ix, int32_t validate, hipStream_t stream) {
  hipLaunchKernelGGL(k_heads, dim3(d.n_heads), dim3(kThreads), 0, stream, d, ix, validate);
  return hipGetLastError();
}

hipError_t launch_index_items(const sa_pattern_desc& d, const sa_index& ix, int32_t fill, int32_t validate,
                              hipStream_t stream) {
  const int64_t items = (int64_t)ix.n_heads * ix.n_row_blocks;
  ItemConsts kc{};
  kc.nwords = ((d.S - 1) >> 5) + 1;
  const size_t bitmaps = 2 * sizeof(uint32_t) * (size_t)kc.nwords;
  kc.dcap = kDsh;  // staged diagonal offsets (count pass) / gathered-column stage (fill pass)
  kc.nbq = 0;
  kc.rb_per_br = 1;
  kc.wpb = 1;
  kc.wpb_shift = 0;
  kc.bs = 64;
  if (d.block_mask != nullptr) {
    kc.bs = d.block_size;
    kc.nbq = (d.S + d.block_size - 1) / d.block_size;
    kc.rb_per_br = d.block_size / ix.row_block;
    kc.wpb = d.block_size / 32;
    kc.wpb_shift = -1;
    for (int s = 0; s < 31; ++s)
      if ((1 << s) == kc.wpb) kc.wpb_shift = s;
  }
  kc.nst = 0;
  kc.rb_per_st = 1;
  if (d.stripe_ptr != nullptr) {
    kc.nst = (d.S + d.stripe_rows - 1) / d.stripe_rows;
    kc.rb_per_st = d.stripe_rows / ix.row_block;
  }
  const size_t lds = bitmaps + sizeof(int32_t) * (size_t)kDsh;
  if (lds > kDefaultLds) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_items),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const unsigned list_grid = (unsigned)((items + kListWaves - 1) / kListWaves);
  hipLaunchKernelGGL(k_items_lists, dim3(list_grid), dim3(64 * kListWaves), 0, stream, d, ix, fill, validate, kc,
                     (int32_t)items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned gen_grid = (unsigned)((items + kGenBatch - 1) / kGenBatch);
  hipLaunchKernelGGL(k_items, dim3(gen_grid), dim3(kThreads), lds, stream, d, ix, fill, validate, kc, (int32_t)items);
  return hipGetLastError();
}

hipError_t launch_index_scan(const sa_index& ix, hipStream_t stream) {
  const int64_t items = (int64_t)ix.n_heads * ix.n_row_blocks;
  const unsigned chunks = (unsigned)((items + kScanChunk - 1) / kScanChunk);
  hipLaunchKernelGGL(k_scan_local, dim3(chunks, 3), dim3(kThreads), 0, stream, ix.seg_ptr, ix.bcol_ptr, ix.col_ptr,
                     items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (chunks > 1) {
    hipLaunchKernelGGL(k_scan_offset, dim3(chunks, 3), dim3(kThreads), 0, stream, ix.seg_ptr, ix.bcol_ptr,
                       ix.col_ptr, items);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_scan_fix, dim3(1), dim3(kThreads), 0, stream, ix.seg_ptr, ix.bcol_ptr, ix.col_ptr, items,
                     ix.run_ptr, ix.n_heads, ix.status);
  return hipGetLastError();
}

hipError_t launch_index_heads_fill(const sa_pattern_desc& d, const sa_index& ix, hipStream_t stream) {
  const int32_t nwords = ((d.S - 1) >> 5) + 1;
  hipLaunchKernelGGL(k_heads_fill, dim3(d.n_heads), dim3(kThreads), sizeof(uint32_t) * (size_t)nwords, stream, d,
                     ix, nwords);
  return hipGetLastError();
}

}  // namespace sa
