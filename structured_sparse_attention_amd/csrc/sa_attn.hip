// sa_attn.hip -- structured sparse prefill attention forward on gfx950.
//
// What is computed (Pith review of "DAM: Dynamic Attention Mask for Long-Context
// Large Language Model Inference Acceleration", Referee Report Summary and "What
// carries the argument"): logits Q K^T / sqrt(d_k), the structured mask applied
// before the softmax so that non-retained pairs get no weight, softmax, times V.
// Only retained pairs are computed ("Circularity Check" step 2: cost ~ retained
// keys per query), using the canonical index of include/sa.h.
//
// Work item: (batch, query head, row block of BM rows).  One workgroup of BM/32
// waves; wave w owns query rows b0 + 32w .. +31.  Keys are processed in tiles of
// BN = 64:
//   segment phase  contiguous key tiles over each interval of U (the columns the
//                  diagonals touch); per-lane 64-bit key masks from the diagonal
//                  runs, the in-segment columns (bcols) and causality;
//   gathered phase tiles of 64 columns from the gathered list (cols): K/V rows are
//                  gathered row by row; only causality can mask (the list is sorted,
//                  so the retained keys of a row are a prefix of the tile).
// Products run on MFMA.  The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 (or 32x32x2_f32): lane l then holds one query row
// (l % 32) and 32 of its keys, so the row max and row sum are in-lane reductions
// plus one exchange between lane l and l^32 (v_permlane32_swap).  O^T = V^T P^T
// reuses the score layout as the B operand directly; V is stored transposed in LDS
// with the key order inside each 16-key group permuted (bits 2 and 3 swapped) so
// that each lane's 8 keys are 16 contiguous bytes.  Softmax is the online
// (running max / running sum) form in fp32 with exp2 and a pre-multiplied
// log2(e) scale; the O rescale is skipped when no row max moved.
// Block order: row blocks in descending order (longest causal work first), and,
// when batch*hkv is a multiple of 8, the work of one kv head stays on one XCD
// (workgroup k runs on XCD k % 8), so one XCD's L2 serves one kv head's K/V.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 64;

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, hq, hkv, S, nb, BM;
  float scale_log2;  // softmax scale * log2(e)
  const int64_t* seg_ptr;
  const int32_t* seg_lo;
  const int32_t* seg_hi;
  const int64_t* bcol_ptr;
  const int32_t* bcol_idx;
  const int64_t* col_ptr;
  const int32_t* col_idx;
  const int32_t* run_ptr;
  const int32_t* run_lo;
  const int32_t* run_hi;
};

__device__ inline uint64_t prefix_mask(int n) {  // bits [0, n), n clamped to [0, 64]
  return n <= 0 ? 0ull : (n >= 64 ? ~0ull : ((1ull << n) - 1ull));
}
__device__ inline uint64_t range_mask(int a, int b) {  // bits [a, b], 0 <= a <= b <= 63
  return (~0ull >> (63 - b)) & (~0ull << a);
}

// max/sum of a value and its copy in lane l ^ 32
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// a * b - c as two rounded operations (no fused multiply-add)
__device__ inline float mul_then_sub(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b - c;
}

// position of key kk inside the transposed V tile: bits 2 and 3 swapped
__device__ inline int vt_pos(int kk) { return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1); }

template <int D, int BM, bool BF16>
struct Cfg {
  static constexpr int NW = BM / 32;
  static constexpr int T = 64 * NW;
  static constexpr int QS = BF16 ? D / 16 : D / 2;  // MFMA k-steps over d
  static constexpr int OB = D / 32;                  // 32-wide d blocks of the output
  // LDS strides in elements
  static constexpr int KS = BF16 ? D + 8 : D + 1;    // K tile [BN][KS]
  static constexpr int VS = BF16 ? BN + 8 : D + 4;   // bf16: V^T [D][VS]; f32: V [BN][VS]
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = BF16 ? D * VS : BN * VS;
  using elem = typename std::conditional<BF16, unsigned short, float>::type;
};

// Work-item decode: blockIdx -> (batch, head, row block).
__device__ inline void decode_item(const Params& p, int& b, int& h, int& rb) {
  const int k = blockIdx.x;
  const int G = p.B * p.hkv, hpg = p.hq / p.hkv;
  if ((G & 7) == 0) {
    const int x = k & 7, s = k >> 3;
    const int gper = G >> 3;
    const int per_rb = gper * hpg;
    rb = p.nb - 1 - s / per_rb;
    const int rest = s % per_rb;
    const int g = x + 8 * (rest / hpg);
    b = g / p.hkv;
    h = (g % p.hkv) * hpg + rest % hpg;
  } else {
    const int per_rb = p.B * p.hq;
    rb = p.nb - 1 - k / per_rb;
    const int rest = k % per_rb;
    b = rest / p.hq;
    h = rest % p.hq;
  }
}

template <int D, int BM, bool BF16>
__global__ void __launch_bounds__(2 * BM) k_attn(Params p) {  // 2*BM threads = BM/32 waves
  using C = Cfg<D, BM, BF16>;
  using E = typename C::elem;
  __shared__ __attribute__((aligned(16))) E Ks[C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) E Vs[C::V_ELEMS];
  __shared__ int32_t cols_sh[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  int b, h, rb;
  decode_item(p, b, h, rb);
  const int S = p.S;
  const int b0 = rb * BM, b1 = min(S, b0 + BM) - 1;
  const int i = b0 + wave * 32 + r32;  // this lane's query row
  const bool row_ok = i <= b1;
  const int kvh = h / (p.hq / p.hkv);

  const E* Qg = static_cast<const E*>(p.q) + ((int64_t)(b * p.hq + h) * S) * D;
  const E* Kg = static_cast<const E*>(p.k) + ((int64_t)(b * p.hkv + kvh) * S) * D;
  const E* Vg = static_cast<const E*>(p.v) + ((int64_t)(b * p.hkv + kvh) * S) * D;

  // ---- Q fragment (B operand of S^T = K Q^T): row r32, d slice per k-step
  using QF = typename std::conditional<BF16, bf16x8, float>::type;
  QF qf[C::QS];
  if constexpr (BF16) {
#pragma unroll
    for (int s = 0; s < C::QS; ++s) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row_ok) u = *reinterpret_cast<const uint4*>(Qg + (int64_t)i * D + 16 * s + 8 * g);
      qf[s] = *reinterpret_cast<bf16x8*>(&u);
    }
  } else {
#pragma unroll
    for (int s = 0; s < C::QS; ++s) qf[s] = row_ok ? Qg[(int64_t)i * D + 2 * s + g] : 0.0f;
  }

  f32x16 oacc[C::OB];
#pragma unroll
  for (int x = 0; x < C::OB; ++x)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[x][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int64_t item = (int64_t)h * p.nb + rb;
  const int32_t r0 = p.run_ptr[h], r1 = p.run_ptr[h + 1];

  // ---- one tile: keys given by key_of(kk) (kk in [0, 64)), per-lane mask `m`
  auto load_tile = [&](auto key_of, int nvalid) {
    if constexpr (BF16) {
      constexpr int CPR = D / 8;  // 16-byte chunks per row
      for (int x = tid; x < BN * CPR; x += C::T) {
        const int kk = x / CPR, c = x % CPR;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (kk < nvalid) {
          const int j = key_of(kk);
          if (j < S) u = *reinterpret_cast<const uint4*>(Kg + (int64_t)j * D + 8 * c);
        }
        *reinterpret_cast<uint4*>(&Ks[kk * C::KS + 8 * c]) = u;
      }
      for (int x = tid; x < (BN / 4) * CPR; x += C::T) {
        const int c = x % CPR, q4 = x / CPR;
        uint4 u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kk = 4 * q4 + t;
          u[t] = make_uint4(0, 0, 0, 0);
          if (kk < nvalid) {
            const int j = key_of(kk);
            if (j < S) u[t] = *reinterpret_cast<const uint4*>(Vg + (int64_t)j * D + 8 * c);
          }
        }
        const int pos = vt_pos(4 * q4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int wsel = e >> 1, sh = (e & 1) * 16;
          uint32_t a0 = ((&u[0].x)[wsel] >> sh) & 0xffffu, a1 = ((&u[1].x)[wsel] >> sh) & 0xffffu;
          uint32_t a2 = ((&u[2].x)[wsel] >> sh) & 0xffffu, a3 = ((&u[3].x)[wsel] >> sh) & 0xffffu;
          uint2 w2 = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
          *reinterpret_cast<uint2*>(&Vs[(8 * c + e) * C::VS + pos]) = w2;
        }
      }
    } else {
      constexpr int CPR = D / 4;  // float4 chunks per row
      for (int x = tid; x < BN * CPR; x += C::T) {
        const int kk = x / CPR, c = x % CPR;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (kk < nvalid) {
          const int j = key_of(kk);
          if (j < S) {
            kv = *reinterpret_cast<const float4*>(Kg + (int64_t)j * D + 4 * c);
            vv = *reinterpret_cast<const float4*>(Vg + (int64_t)j * D + 4 * c);
          }
        }
        Ks[kk * C::KS + 4 * c + 0] = kv.x;
        Ks[kk * C::KS + 4 * c + 1] = kv.y;
        Ks[kk * C::KS + 4 * c + 2] = kv.z;
        Ks[kk * C::KS + 4 * c + 3] = kv.w;
        *reinterpret_cast<float4*>(&Vs[kk * C::VS + 4 * c]) = vv;
      }
    }
  };

  auto compute_tile = [&](uint64_t m) {
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
      if constexpr (BF16) {
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + r32) * C::KS + 16 * s + 8 * g]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
          const float kf = Ks[(kb * 32 + r32) * C::KS + 2 * s + g];
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf, qf[s], sacc[kb], 0, 0, 0);
        }
      }
    }
    // mask: value v of block kb is key kb*32 + 8*(v/4) + 4*g + v%4
    const bool full = (m == ~0ull);
    if (!__all(full)) {
      const uint64_t mg = m >> (4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!((mg >> (kb * 32 + 8 * (v >> 2) + (v & 3))) & 1ull)) sacc[kb][v] = -INFINITY;
    }
    // online softmax (log2 domain)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // bf16: one fma per score.  fp32: scale first, so the row maximum maps to exp2(0) = 1 exactly.
        const float arg = BF16 ? __builtin_fmaf(sacc[kb][v], p.scale_log2, -m_use)
                               : mul_then_sub(sacc[kb][v], p.scale_log2, m_use);
        const float e = __builtin_amdgcn_exp2f(arg);
        sacc[kb][v] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int x = 0; x < C::OB; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[x][v] *= alpha;
    }
    m_run = m_new;
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (BF16) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          bf16x8 pf;
#pragma unroll
          for (int t = 0; t < 8; ++t) pf[t] = (__bf16)sacc[kb][8 * mm + t];
#pragma unroll
          for (int x = 0; x < C::OB; ++x) {
            const bf16x8 vf =
                *reinterpret_cast<const bf16x8*>(&Vs[(32 * x + r32) * C::VS + kb * 32 + 16 * mm + 8 * g]);
            oacc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[x], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
#pragma unroll
          for (int x = 0; x < C::OB; ++x) {
            const float vf = Vs[key * C::VS + 32 * x + r32];
            oacc[x] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf, sacc[kb][v], oacc[x], 0, 0, 0);
          }
        }
      }
    }
  };

  // ---------------- segment phase
  {
    int64_t bp = p.bcol_ptr[item];
    const int64_t bp_end = p.bcol_ptr[item + 1];
    const int64_t s0 = p.seg_ptr[item], s1 = p.seg_ptr[item + 1];
    for (int64_t s = s0; s < s1; ++s) {
      const int slo = p.seg_lo[s], shi = p.seg_hi[s];
      for (int j0 = slo; j0 <= shi; j0 += BN) {
        const int nvalid = min(BN, shi - j0 + 1);
        // in-segment columns of this tile (sorted list, consumed in order)
        uint64_t xin = 0;
        while (bp < bp_end) {
          const int c = p.bcol_idx[bp];
          if (c >= j0 + nvalid) break;
          xin |= 1ull << (c - j0);
          ++bp;
        }
        // per-lane key mask: diagonals, in-segment columns, valid range, causality.
        // Runs that can meet this tile have offsets in [b0 - j0 - 63, b1 - j0]; runs are sorted and
        // disjoint, so the first candidate is found by binary search on run_hi.
        const int omin = b0 - j0 - (BN - 1), omax = b1 - j0;
        int32_t rf = r0, rl = r1;
        while (rf < rl) {
          const int32_t mid = (rf + rl) >> 1;
          if (p.run_hi[mid] < omin) rf = mid + 1;
          else rl = mid;
        }
        uint64_t m = 0;
        const int base = i - j0;  // key kk of this lane's row has offset base - kk
        for (int32_t r = rf; r < r1; ++r) {
          const int lo = p.run_lo[r];
          if (lo > omax) break;
          const int hi = p.run_hi[r];
          const int a = max(0, base - hi), e = min(BN - 1, base - lo);
          if (a <= e) m |= range_mask(a, e);
        }
        m |= xin;
        m &= prefix_mask(nvalid) & prefix_mask(base + 1);
        if (!row_ok) m = 0;
        __syncthreads();
        load_tile([&](int kk) { return j0 + kk; }, nvalid);
        __syncthreads();
        compute_tile(m);
      }
    }
  }
  // ---------------- gathered phase
  {
    const int64_t c0 = p.col_ptr[item], c1 = p.col_ptr[item + 1];
    for (int64_t pc = c0; pc < c1; pc += BN) {
      const int nvalid = (int)min((int64_t)BN, c1 - pc);
      __syncthreads();
      if (tid < BN) cols_sh[tid] = tid < nvalid ? p.col_idx[pc + tid] : 0;
      __syncthreads();
      load_tile([&](int kk) { return cols_sh[kk]; }, nvalid);
      __syncthreads();
      uint64_t m = 0;
      if (row_ok) {
        int cnt;
        if (cols_sh[nvalid - 1] <= i) {
          cnt = nvalid;
        } else {
          int lo = 0, hi = nvalid;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (cols_sh[mid] <= i) lo = mid + 1;
            else hi = mid;
          }
          cnt = lo;
        }
        m = prefix_mask(cnt);
      }
      compute_tile(m);
    }
  }

  // ---------------- epilogue
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
    E* Og = static_cast<E*>(p.o) + ((int64_t)(b * p.hq + h) * S + i) * D;
#pragma unroll
    for (int x = 0; x < C::OB; ++x)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * x + 8 * qd + 4 * g;
        if constexpr (BF16) {
          __bf16 t4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) t4[e] = (__bf16)(oacc[x][4 * qd + e] * inv);
          *reinterpret_cast<uint2*>(Og + d0) = *reinterpret_cast<uint2*>(t4);
        } else {
          float4 f = make_float4(oacc[x][4 * qd] * inv, oacc[x][4 * qd + 1] * inv, oacc[x][4 * qd + 2] * inv,
                                 oacc[x][4 * qd + 3] * inv);
          *reinterpret_cast<float4*>(Og + d0) = f;
        }
      }
    if (p.lse != nullptr && g == 0) {
      p.lse[(int64_t)(b * p.hq + h) * S + i] =
          l_tot > 0.0f ? m_run * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, int BM, bool BF16>
hipError_t launch_t(const Params& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.B * p.hq * p.nb;
  k_attn<D, BM, BF16><<<dim3((unsigned)blocks), dim3(Cfg<D, BM, BF16>::T), 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_bm(const Params& p, hipStream_t stream) {
  return p.BM == 64 ? launch_t<D, 64, BF16>(p, stream) : launch_t<D, 128, BF16>(p, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.B = a.batch;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.S = a.S;
  p.nb = a.idx->n_row_blocks;
  p.BM = a.idx->row_block;
  p.scale_log2 = a.scale * 1.44269504088896340736f;
  p.seg_ptr = a.idx->seg_ptr;
  p.seg_lo = a.idx->seg_lo;
  p.seg_hi = a.idx->seg_hi;
  p.bcol_ptr = a.idx->bcol_ptr;
  p.bcol_idx = a.idx->bcol_idx;
  p.col_ptr = a.idx->col_ptr;
  p.col_idx = a.idx->col_idx;
  p.run_ptr = a.idx->run_ptr;
  p.run_lo = a.idx->run_lo;
  p.run_hi = a.idx->run_hi;
  const bool bf = a.dtype == SA_DTYPE_BF16;
  if (a.head_dim == 64) return bf ? launch_bm<64, true>(p, stream) : launch_bm<64, false>(p, stream);
  return bf ? launch_bm<128, true>(p, stream) : launch_bm<128, false>(p, stream);
}

}  // namespace sa
