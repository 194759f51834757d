// sa_plan.hip -- work plan of the key-sliced attention schedule on gfx950.
//
// Why: the cost of the masked attention is the retained keys per query ("Circularity Check",
// step 2, of the Pith review of "DAM: Dynamic Attention Mask for Long-Context Large Language
// Model Inference Acceleration"), and with block-sparse or scattered-column masks each retained
// 64 x 64 tile needs its own 64 K and V rows.  One kv head's K/V at S = 65536, d = 128 is 32 MiB:
// eight times one XCD's 4 MiB L2, so tiles fetched for one row block are evicted long before the
// next row block that needs them asks again.  Cutting the key axis into eight slices of S/8 keys
// (4 MiB of K/V each) and running every slice of a kv head on its own XCD keeps each XCD's
// working set inside its L2.
//
// The plan (four launches, all on the caller's stream, before the attention kernel):
//   k_plan_zero     clears the queue heads, bucket counters and per-item merge counters;
//   k_plan_items    one wave per (query head, row block) item: decides whether the item is
//                   sliced (at least kSliceMinCols gathered columns spread over two or more
//                   slices), finds each slice's sub-ranges of the item's gathered columns,
//                   segments and in-segment columns by binary search (lane s: slice s), and
//                   stages one unit per slice that holds keys; counts units per (kv head, slice);
//   k_plan_buckets  one workgroup: the position of every (kv group, slice) bucket in its XCD's
//                   queue.  XCD x takes, in order, kv group g's slice (x + g) mod 8 for
//                   g = 0, 1, ...: each XCD sees every slice once per eight groups (the work
//                   per slice falls with the slice index, so this balances the XCDs) and reads
//                   one 4 MiB slice at a time;
//   k_plan_scatter  one thread per (batch, item): copies the item's units into their buckets.
// Unsliced items go to the bucket of the slice that holds their last row (their band tiles).
#include "sa_internal.h"

namespace sa {

namespace {

struct PlanHead {
  int32_t pop[kMaxSlices];    // next queue position per XCD (attention kernel)
  int32_t qbase[kMaxSlices];  // first unit of each XCD's queue
  int32_t qlen[kMaxSlices];   // units in each XCD's queue
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// first index in [lo, hi) with a[index] >= x (a sorted ascending)
__device__ inline int64_t lower_bound_ge(const int32_t* a, int64_t lo, int64_t hi, int32_t x) {
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

struct PlanParams {
  int32_t S, BM, nb, hq, hkv, B, KR, ns, G;
  int64_t items;
  int64_t slots_per_head;
  const int64_t* seg_ptr;
  const int32_t* seg_lo;
  const int32_t* seg_hi;
  const int64_t* bcol_ptr;
  const int32_t* bcol_idx;
  const int64_t* col_ptr;
  const int32_t* col_idx;
  PlanHead* head;
  int32_t* counts;   // [hkv][kMaxSlices]
  int32_t* fills;    // [G][kMaxSlices]
  int32_t* bbase;    // [G][kMaxSlices], relative to the XCD's queue start
  int32_t* nunits;   // [items] (in the stage area's tail)
  AttnUnit* stage;   // [items][kMaxSlices]
  AttnUnit* units;   // [max_units]
};

__global__ void __launch_bounds__(256) k_plan_zero(int32_t* p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = 0;
}

__global__ void __launch_bounds__(256) k_plan_items(PlanParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= p.items) return;
  const int h = (int)(item / p.nb), rb = (int)(item % p.nb);
  const int b1 = min(p.S, (rb + 1) * p.BM) - 1;
  const int hs = b1 / p.KR;  // slice of the item's last row
  const int kvh = h / (p.hq / p.hkv);
  const int64_t c0 = p.col_ptr[item], c1 = p.col_ptr[item + 1];
  const int64_t s0 = p.seg_ptr[item], s1 = p.seg_ptr[item + 1];
  const int64_t q0 = p.bcol_ptr[item], q1 = p.bcol_ptr[item + 1];
  bool sliced = false;
  if (hs > 0 && c1 - c0 >= kSliceMinCols) sliced = (p.col_idx[c0] / p.KR) != (p.col_idx[c1 - 1] / p.KR);
  AttnUnit* st = p.stage + item * kMaxSlices;
  if (!sliced) {
    if (lane == 0) {
      AttnUnit u;
      u.b = 0;
      u.item = (int32_t)item;
      u.klo = 0;
      u.khi = p.S - 1;
      u.part = 0;
      u.nparts = 1;
      u.slice = hs;
      u.pad = 0;
      u.ca = c0;
      u.cb = c1;
      u.sa = s0;
      u.sb = s1;
      u.bp = q0;
      st[0] = u;
      p.nunits[item] = 1;
      atomicAdd(&p.counts[kvh * kMaxSlices + hs], 1);
    }
    return;
  }
  // lane s < kMaxSlices: the sub-ranges of slice s = keys [s * KR, (s + 1) * KR)
  const int s = lane;
  bool nonempty = false;
  AttnUnit u;
  if (s <= hs) {
    const int32_t klo = s * p.KR, khi_ex = (s + 1) * p.KR;
    u.ca = lower_bound_ge(p.col_idx, c0, c1, klo);
    u.cb = lower_bound_ge(p.col_idx, u.ca, c1, khi_ex);
    u.sa = lower_bound_ge(p.seg_hi, s0, s1, klo);      // first segment reaching the slice
    u.sb = lower_bound_ge(p.seg_lo, u.sa, s1, khi_ex);  // first segment starting past it
    u.bp = lower_bound_ge(p.bcol_idx, q0, q1, klo);
    u.klo = klo;
    u.khi = min(khi_ex, p.S) - 1;
    nonempty = (u.ca < u.cb) || (u.sa < u.sb);
  }
  const uint64_t mask = __ballot(nonempty);
  const int n = __popcll(mask);
  if (nonempty) {
    u.b = 0;
    u.item = (int32_t)item;
    u.part = __popcll(mask & ((1ull << s) - 1ull));
    u.nparts = n;
    u.slice = s;
    u.pad = 0;
    st[u.part] = u;
    atomicAdd(&p.counts[kvh * kMaxSlices + s], 1);
  }
  if (lane == 0) p.nunits[item] = n;
}

// One workgroup of kMaxSlices waves; wave x lays out XCD x's queue: buckets (g, (x + g) mod 8)
// for g = 0 .. G-1 (slices past the last one are empty), 64 groups per step with a wave-wide scan.
__global__ void __launch_bounds__(64 * kMaxSlices) k_plan_buckets(PlanParams p) {
  __shared__ int32_t qlen_sh[kMaxSlices];
  const int lane = threadIdx.x & 63, x = threadIdx.x >> 6;
  int32_t carry = 0;
  for (int g0 = 0; g0 < p.G; g0 += 64) {
    const int g = g0 + lane;
    const int s = (x + g) % kMaxSlices;
    int32_t c = 0;
    if (g < p.G && s < p.ns) c = p.counts[(g % p.hkv) * kMaxSlices + s];
    // inclusive scan over the wave
    int32_t v = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(v, o, 64);
      if (lane >= o) v += t;
    }
    if (g < p.G && s < p.ns) p.bbase[g * kMaxSlices + s] = carry + v - c;
    carry += __shfl(v, 63, 64);
  }
  if (lane == 0) qlen_sh[x] = carry;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t pos = 0;
    for (int q = 0; q < kMaxSlices; ++q) {
      p.head->qbase[q] = pos;
      p.head->qlen[q] = qlen_sh[q];
      p.head->pop[q] = 0;
      pos += qlen_sh[q];
    }
  }
}

__global__ void __launch_bounds__(256) k_plan_scatter(PlanParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.items * p.B) return;
  const int b = (int)(t / p.items);
  const int64_t item = t % p.items;
  const int h = (int)(item / p.nb);
  const int g = b * p.hkv + h / (p.hq / p.hkv);
  const int n = p.nunits[item];
  const AttnUnit* st = p.stage + item * kMaxSlices;
  for (int k = 0; k < n; ++k) {
    AttnUnit u = st[k];
    u.b = b;
    const int s = u.slice;
    const int x = ((s - g) % kMaxSlices + kMaxSlices) % kMaxSlices;
    const int32_t pos = p.head->qbase[x] + p.bbase[g * kMaxSlices + s] + atomicAdd(&p.fills[g * kMaxSlices + s], 1);
    p.units[pos] = u;
  }
}

}  // namespace

PlanLayout plan_layout(int32_t batch, int32_t hq, int32_t hkv, int32_t S, int32_t head_dim, int32_t dtype,
                       int32_t row_block) {
  PlanLayout L{};
  if (dtype != SA_DTYPE_BF16 || row_block != 64) return L;
  const int64_t nb = (S + 63) / 64;
  L.KR = (int32_t)(64 * ((((int64_t)S + kMaxSlices - 1) / kMaxSlices + 63) / 64));
  L.ns = (int32_t)((S + L.KR - 1) / L.KR);
  L.G = batch * hkv;
  L.items = (int64_t)hq * nb;
  // partial slots: one per (item, slice up to the item's last row); slice of row block rb = rb / q
  const int64_t q = L.KR / 64;
  int64_t C = 0;
  for (int64_t s = 0; s * q < nb; ++s) C += (s + 1) * std::min(q, nb - s * q);
  L.slots_per_head = C;
  L.max_units = (int64_t)batch * hq * C;
  const int OB = head_dim / 32;
  L.slot_bytes = 2 /* waves */ * 64 /* lanes */ * ((size_t)OB * 16 + 4) * sizeof(float);  // accumulators, (m, l, -, -)
  size_t off = 0;
  L.head = off;
  off = align256(off + sizeof(PlanHead));
  L.counts = off;
  off = align256(off + (size_t)hkv * kMaxSlices * sizeof(int32_t));
  L.fills = off;
  off = align256(off + (size_t)L.G * kMaxSlices * sizeof(int32_t));
  L.cnt = off;
  off = align256(off + (size_t)batch * L.items * sizeof(int32_t));
  L.bbase = off;  // everything before here is zeroed by each plan
  off = align256(off + (size_t)L.G * kMaxSlices * sizeof(int32_t));
  L.stage = off;
  off = align256(off + (size_t)L.items * kMaxSlices * sizeof(AttnUnit) + (size_t)L.items * sizeof(int32_t));
  L.units = off;
  off = align256(off + (size_t)L.max_units * sizeof(AttnUnit));
  L.partials = off;
  off = align256(off + (size_t)L.max_units * L.slot_bytes);
  L.total = off;
  return L;
}

hipError_t launch_plan(const AttnArgs& a, const PlanLayout& L, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  PlanParams p;
  p.S = a.S;
  p.BM = a.idx->row_block;
  p.nb = a.idx->n_row_blocks;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.B = a.batch;
  p.KR = L.KR;
  p.ns = L.ns;
  p.G = L.G;
  p.items = L.items;
  p.slots_per_head = L.slots_per_head;
  p.seg_ptr = a.idx->seg_ptr;
  p.seg_lo = a.idx->seg_lo;
  p.seg_hi = a.idx->seg_hi;
  p.bcol_ptr = a.idx->bcol_ptr;
  p.bcol_idx = a.idx->bcol_idx;
  p.col_ptr = a.idx->col_ptr;
  p.col_idx = a.idx->col_idx;
  p.head = reinterpret_cast<PlanHead*>(ws + L.head);
  p.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  p.fills = reinterpret_cast<int32_t*>(ws + L.fills);
  p.bbase = reinterpret_cast<int32_t*>(ws + L.bbase);
  p.stage = reinterpret_cast<AttnUnit*>(ws + L.stage);
  p.nunits = reinterpret_cast<int32_t*>(ws + L.stage + (size_t)L.items * kMaxSlices * sizeof(AttnUnit));
  p.units = reinterpret_cast<AttnUnit*>(ws + L.units);
  const int64_t nzero = (int64_t)(L.bbase / sizeof(int32_t));
  k_plan_zero<<<dim3((unsigned)std::min<int64_t>((nzero + 255) / 256, 2048)), dim3(256), 0, stream>>>(
      reinterpret_cast<int32_t*>(ws), nzero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_plan_items<<<dim3((unsigned)((L.items + 3) / 4)), dim3(256), 0, stream>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_plan_buckets<<<dim3(1), dim3(64 * kMaxSlices), 0, stream>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nt = L.items * a.batch;
  k_plan_scatter<<<dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace sa
