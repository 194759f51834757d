// sa_decode.hip -- structured sparse attention for one new query row per sequence
// (decode against a K/V cache) on gfx950.
//
// What is computed (Pith review of "DAM: Dynamic Attention Mask for Long-Context
// Large Language Model Inference Acceleration", Referee Report Summary and "What
// carries the argument"): the query of sequence b sits at position t = pos[b]; it
// attends to the cache rows j <= t that the mask retains for row t (masked logits
// get no weight), with softmax(q K^T / sqrt(d_k)) V over those rows.  This is row t
// of the prefill output when Q[b][h][t] is the given query, so the same index
// serves both: the item (h, t / BM) lists the key columns of row t's block.
//
// Work: one workgroup of eight waves per (sequence, query head).  Candidate keys are
// the segment columns <= t (retained iff (t - j) is a diagonal offset of the head or
// j is an in-segment column of the item) and the gathered columns <= t.  The waves
// take interleaved batches of 64 candidates; each lane tests one candidate, and the
// retained keys are compacted into a per-wave queue in LDS, so that the work below
// always runs on full groups of 64 retained keys (a far diagonal leaves one key in
// its 64-wide segment).  For a group each lane holds one key: it reads its K row (a
// full row per lane) and forms q . k against the query kept in its registers; the
// group's scores update the wave's running max and sum (exp2 domain).  P.V then runs
// with the lanes over head dimensions: the group's (key, p) pairs are read back from
// LDS and 32 V rows are loaded at once (coalesced rows), every lane accumulating its
// slice.  Decode moves each retained K and V row once and does 4 d flops per row, so
// it is bound by memory latency and bandwidth, not by arithmetic; no MFMA.  The
// waves' partial (max, sum, output) are merged in LDS at the end.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kWaves = 8;

struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* pos;
  int32_t B, hq, hkv, S, nb, BM, nwords;
  float scale_log2;  // softmax scale * log2(e)
  const int64_t* seg_ptr;
  const int32_t* seg_lo;
  const int32_t* seg_hi;
  const int64_t* bcol_ptr;
  const int32_t* bcol_idx;
  const int64_t* col_ptr;
  const int32_t* col_idx;
  const uint32_t* dbits;
};

__device__ inline float dec_wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline float dec_wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// true iff some entry of the sorted list a[lo, hi) equals x
__device__ inline bool in_sorted(const int32_t* a, int64_t lo, int64_t hi, int32_t x) {
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    const int32_t y = a[mid];
    if (y == x) return true;
    if (y < x) lo = mid + 1;
    else hi = mid;
  }
  return false;
}

template <int D, bool BF16>
__global__ void __launch_bounds__(64 * kWaves) k_decode(DecParams p) {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int QW = BF16 ? D / 2 : D;  // query registers: bf16 pairs or fp32 values
  constexpr int DPL = D / 64;           // head dimensions per lane in P.V
  constexpr int VB = 32;                // V rows loaded at once
  __shared__ float m_sh[kWaves], l_sh[kWaves];
  __shared__ float o_sh[kWaves][D];
  __shared__ int32_t kq[kWaves][128];  // per-wave queue of retained keys
  __shared__ float kp[kWaves][64];     // probabilities of the group being processed

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x / p.hq, h = blockIdx.x % p.hq;
  const int kvh = h / (p.hq / p.hkv);
  const int S = p.S;
  const int t = p.pos[b];
  E* Og = static_cast<E*>(p.o) + ((int64_t)b * p.hq + h) * D;
  if (t < 0 || t >= S) {  // no valid query row: zero output, -inf lse
    for (int d = threadIdx.x; d < D; d += 64 * kWaves) Og[d] = (E)0;
    if (threadIdx.x == 0 && p.lse != nullptr) p.lse[(int64_t)b * p.hq + h] = -INFINITY;
    return;
  }
  const E* Kg = static_cast<const E*>(p.k) + ((int64_t)b * p.hkv + kvh) * S * (int64_t)D;
  const E* Vg = static_cast<const E*>(p.v) + ((int64_t)b * p.hkv + kvh) * S * (int64_t)D;

  // the query, whole, in every lane
  uint32_t qw[QW];
  {
    const uint32_t* qsrc = reinterpret_cast<const uint32_t*>(static_cast<const E*>(p.q) + ((int64_t)b * p.hq + h) * D);
#pragma unroll
    for (int c = 0; c < QW; c += 4) {
      const uint4 u = *reinterpret_cast<const uint4*>(qsrc + c);
      qw[c] = u.x;
      qw[c + 1] = u.y;
      qw[c + 2] = u.z;
      qw[c + 3] = u.w;
    }
  }

  const int rb = t / p.BM;
  const int64_t item = (int64_t)h * p.nb + rb;
  const uint32_t* dbh = p.dbits + (int64_t)h * p.nwords;
  const int64_t bc0 = p.bcol_ptr[item], bc1 = p.bcol_ptr[item + 1];

  float m_run = -INFINITY;  // running max of the wave's scores (log2 domain), wave-uniform
  float l_lane = 0.0f;      // this lane's share of the running sum
  float oacc[DPL];
#pragma unroll
  for (int x = 0; x < DPL; ++x) oacc[x] = 0.0f;
  int qn = 0;  // keys waiting in kq[wave] (wave-uniform)

  // the first n (1..64) keys of the queue: lane l takes key kq[wave][l]
  auto group = [&](int n) {
    const bool keep = lane < n;
    const int32_t j = keep ? kq[wave][lane] : 0;
    float x = -INFINITY;
    if (keep) {
      const uint4* krow = reinterpret_cast<const uint4*>(Kg + (int64_t)j * D);
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < QW / 4; ++c) {
        const uint4 kv = krow[c];
        const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (BF16) {
            acc = __builtin_fmaf(bf16_lo(qw[4 * c + e]), bf16_lo(kk[e]), acc);
            acc = __builtin_fmaf(bf16_hi(qw[4 * c + e]), bf16_hi(kk[e]), acc);
          } else {
            acc = __builtin_fmaf(__uint_as_float(qw[4 * c + e]), __uint_as_float(kk[e]), acc);
          }
        }
      }
      x = acc * p.scale_log2;
    }
    const float gmax = dec_wave_max(x);  // finite: lane 0 holds a key
    if (gmax > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - gmax);  // exp2(-inf) = 0 on the first group
      l_lane *= alpha;
#pragma unroll
      for (int e = 0; e < DPL; ++e) oacc[e] *= alpha;
      m_run = gmax;
    }
    const float pj = keep ? __builtin_amdgcn_exp2f(x - m_run) : 0.0f;
    l_lane += pj;
    kp[wave][lane] = pj;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's LDS writes are done before it reads them
    // P.V with the lanes over head dimensions: lane owns dimensions [DPL * lane, DPL * lane + DPL)
    for (int u0 = 0; u0 < n; u0 += VB) {
      float ps[VB];
      if constexpr (BF16) {
        uint32_t w[VB];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const bool live = u0 + u < n;
          const int32_t jj = live ? kq[wave][u0 + u] : 0;
          ps[u] = live ? kp[wave][u0 + u] : 0.0f;
          const E* vrow = Vg + (int64_t)jj * D + DPL * lane;
          if constexpr (DPL == 2) w[u] = live ? *reinterpret_cast<const uint32_t*>(vrow) : 0u;
          else w[u] = live ? (uint32_t)(*reinterpret_cast<const uint16_t*>(vrow)) << 16 : 0u;
        }
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          if constexpr (DPL == 2) {
            oacc[0] = __builtin_fmaf(ps[u], bf16_lo(w[u]), oacc[0]);
            oacc[1] = __builtin_fmaf(ps[u], bf16_hi(w[u]), oacc[1]);
          } else {
            oacc[0] = __builtin_fmaf(ps[u], __uint_as_float(w[u]), oacc[0]);
          }
        }
      } else {
        float w[VB][DPL];
#pragma unroll
        for (int u = 0; u < VB; ++u) {
          const bool live = u0 + u < n;
          const int32_t jj = live ? kq[wave][u0 + u] : 0;
          ps[u] = live ? kp[wave][u0 + u] : 0.0f;
          const E* vrow = Vg + (int64_t)jj * D + DPL * lane;
#pragma unroll
          for (int e = 0; e < DPL; ++e) w[u][e] = live ? vrow[e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < VB; ++u)
#pragma unroll
          for (int e = 0; e < DPL; ++e) oacc[e] = __builtin_fmaf(ps[u], w[u][e], oacc[e]);
      }
    }
  };

  // Candidates in batches of 64 (lane = candidate j, keep = retained for row t): first the
  // segment columns <= t (retained iff (t - j) is a diagonal offset or j is an in-segment
  // column), then the gathered columns <= t (the list ascends, so they are a prefix).  The
  // retained ones join the queue in order; each full group (and at the end the rest) is
  // processed, the keys beyond it move to the front.  One loop, so that the group code is
  // emitted once.
  const int64_t s0 = p.seg_ptr[item], s1 = p.seg_ptr[item + 1];
  const int64_t c0 = p.col_ptr[item], c1 = p.col_ptr[item + 1];
  int64_t seg = s0;
  int32_t jb = 0, shi = -1;  // current segment's next batch start and end (clipped to t)
  auto open_segment = [&]() {
    while (seg < s1) {
      const int32_t lo = p.seg_lo[seg];
      if (lo > t) {  // segments ascend: none left at or below t
        seg = s1;
        break;
      }
      jb = lo + 64 * wave;
      shi = min(p.seg_hi[seg], t);
      if (jb <= shi) return;
      ++seg;
    }
  };
  open_segment();
  int64_t cb = c0 + 64 * wave;
  bool cols_done = false;
  for (;;) {
    int32_t j = 0;
    bool keep = false, last = false;
    if (seg < s1) {
      j = jb + lane;
      if (j <= shi) {
        const int32_t r = t - j;
        keep = (dbh[r >> 5] >> (r & 31)) & 1u;
        if (!keep && bc1 > bc0) keep = in_sorted(p.bcol_idx, bc0, bc1, j);
      }
      jb += 64 * kWaves;
      if (jb > shi) {
        ++seg;
        open_segment();
      }
    } else if (!cols_done && cb < c1) {
      const int64_t ci = cb + lane;
      j = ci < c1 ? p.col_idx[ci] : S;
      keep = j <= t;
      cb += 64 * kWaves;
      if (__ballot(keep) == 0ull || cb >= c1) cols_done = true;
    } else {
      last = true;
    }
    const uint64_t mask = __ballot(keep);
    if (keep) kq[wave][qn + __popcll(mask & ((1ull << lane) - 1ull))] = j;
    qn += __popcll(mask);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the queue is written before it is read
    if (qn >= 64 || (last && qn > 0)) {
      const int n = min(qn, 64);
      group(n);
      const int32_t rest = lane < qn - n ? kq[wave][n + lane] : 0;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if (lane < qn - n) kq[wave][lane] = rest;
      qn -= n;
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    if (last) break;
  }

  // merge the waves
  const float l_w = dec_wave_sum(l_lane);
  if (lane == 0) {
    m_sh[wave] = m_run;
    l_sh[wave] = l_w;
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) o_sh[wave][DPL * lane + e] = oacc[e];
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_sh[w]);
  float L = 0.0f, f[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    f[w] = (M == -INFINITY || m_sh[w] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_sh[w] - M);
    L += l_sh[w] * f[w];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int d = DPL * lane + e;
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc = __builtin_fmaf(o_sh[w][d], f[w], acc);
    const float y = acc * inv;
    if constexpr (BF16) {
      const __bf16 yb = (__bf16)y;
      Og[d] = *reinterpret_cast<const uint16_t*>(&yb);
    } else {
      Og[d] = y;
    }
  }
  if (lane == 0 && p.lse != nullptr)
    p.lse[(int64_t)b * p.hq + h] = L > 0.0f ? M * 0.69314718055994530942f + logf(L) : -INFINITY;
}

template <int D, bool BF16>
hipError_t launch_decode_t(const DecParams& p, hipStream_t stream) {
  k_decode<D, BF16><<<dim3((unsigned)(p.B * p.hq)), dim3(64 * kWaves), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.pos = a.pos;
  p.B = a.batch;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.S = a.S;
  p.nb = a.idx->n_row_blocks;
  p.BM = a.idx->row_block;
  p.nwords = ((a.S - 1) >> 5) + 1;
  p.scale_log2 = a.scale * 1.44269504088896340736f;
  p.seg_ptr = a.idx->seg_ptr;
  p.seg_lo = a.idx->seg_lo;
  p.seg_hi = a.idx->seg_hi;
  p.bcol_ptr = a.idx->bcol_ptr;
  p.bcol_idx = a.idx->bcol_idx;
  p.col_ptr = a.idx->col_ptr;
  p.col_idx = a.idx->col_idx;
  p.dbits = a.idx->dbits;
  if (a.dtype == SA_DTYPE_BF16) return a.head_dim == 64 ? launch_decode_t<64, true>(p, stream) : launch_decode_t<128, true>(p, stream);
  return a.head_dim == 64 ? launch_decode_t<64, false>(p, stream) : launch_decode_t<128, false>(p, stream);
}

}  // namespace sa
