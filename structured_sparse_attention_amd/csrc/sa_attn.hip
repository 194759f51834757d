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
// Block order (decode_item): kv groups one after another across the whole chip,
// neighbouring row blocks of a group on one XCD, heaviest row blocks first.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
  const uint32_t* dbits;  // [hq][nwords] diagonal offsets as bits
  int32_t nwords;
};

// Values the whole wave shares, loaded through the vector memory path, moved to scalar registers so
// that the tile walk runs on the scalar unit and holds no vector registers.
__device__ inline int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ inline uint64_t prefix_mask(int n) {  // bits [0, n), n clamped to [0, 64]
  return n <= 0 ? 0ull : (n >= 64 ? ~0ull : ((1ull << n) - 1ull));
}
__device__ inline uint64_t range_mask(int a, int b) {  // bits [a, b], 0 <= a <= b <= 63
  return (~0ull >> (63 - b)) & (~0ull << a);
}

// LDS written by some lanes of a wave becomes visible to every lane of that wave
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A work item's list of one or two int32 arrays (segment bounds, in-segment columns), read in
// order by the whole wave.  The wave keeps 64 consecutive entries in its own LDS area and refills
// it when the walk passes its end, so that the walk waits on global memory once per 64 entries, not
// once per entry (a segment change, an in-segment column).  issue() starts the loads of the first
// chunk into registers, so that they travel with other loads; commit() waits for them and stores it.
template <int N, bool REFILL>
struct ListStream {
  const int32_t* src[N];
  int32_t* sh;  // N * 64 entries of this wave's LDS
  int64_t end, base;
  int32_t v[N];
  __device__ void issue(int64_t at) {
    base = at;
    const int64_t q = min(at + (int64_t)(threadIdx.x & 63), max(end - 1, (int64_t)0));
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = end > 0 ? src[k][q] : 0;
  }
  __device__ void commit() {
#pragma unroll
    for (int k = 0; k < N; ++k) sh[k * 64 + (threadIdx.x & 63)] = v[k];
    wave_lds_sync();
  }
  // entry `at` of array k (base <= at < end); wave-uniform.  Past the chunk, the next 64 entries
  // replace it (REFILL), or the entry is read from global memory directly (for a kernel whose loop
  // has no registers to spare for the refill).
  __device__ int32_t get(int k, int64_t at) {
    if (!REFILL && at - base >= 64) return __builtin_amdgcn_readfirstlane(src[k][at]);
    if (at - base >= 64) {
      base = at;
      const int64_t q = min(at + (int64_t)(threadIdx.x & 63), end - 1);
#pragma unroll
      for (int kk = 0; kk < N; ++kk) sh[kk * 64 + (threadIdx.x & 63)] = src[kk][q];
      wave_lds_sync();
    }
    return __builtin_amdgcn_readfirstlane(sh[k * 64 + (int)(at - base)]);
  }
};

// The in-segment columns of a work item, consumed tile by tile in key order.
template <bool REFILL>
struct BcolStream {
  ListStream<1, REFILL> ls;
  int64_t pos;
  // bits (c - j0) of the entries c < j0 + n, consumed
  __device__ uint64_t take(int j0, int n) {
    uint64_t x = 0;
    while (pos < ls.end) {
      const int c = ls.get(0, pos);
      if (c >= j0 + n) break;
      x |= 1ull << (c - j0);
      ++pos;
    }
    return x;
  }
};

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

// LDS banks on gfx950: 64 banks of 4 bytes (256 bytes per cycle).  A 16-byte access is served 16
// lanes at a time, so a conflict-free 16-byte access spreads each group of 16 lanes over 16
// different 16-byte bank groups.
//
// bf16 K and V tiles are stored key-row-major (d values contiguous, 2 * D bytes per row), with
// the 16-byte chunks of row R XOR-swizzled: K chunk c at c ^ kswz(R), V chunk c at c ^ vswz(R).
// - K is read as the A operand of S^T = K Q^T, 16 bytes per lane, lane r (0..31) from key row r:
//   16 consecutive rows must land on 16 different bank groups.  With 256-byte rows (16 chunks)
//   that is chunk ^ (R % 16); with 128-byte rows two rows share the 256 bytes of the banks, so
//   chunk ^ ((R / 2) % 8).
// - V is read with ds_read_b64_tr_b16 (the A operand of O^T = V^T P^T): the 16 lanes of one
//   transposed read take 32 bytes from each of 4 consecutive key rows, and chunk ^ 4 (R % 4)
//   (256-byte rows) or chunk ^ 4 ((R / 2) % 2) (128-byte rows) puts the 8 segments of a half-wave
//   on 8 different 32-byte bank groups.
// Both swizzles depend on R % 16 only, and for R = a + b with a a multiple of 16 and b below it,
// kswz(a + b) = kswz(a) ^ kswz(b) (likewise vswz).
template <int D>
__device__ inline int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ inline int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

template <int D, int BM, bool BF16>
struct Cfg {
  static constexpr int NW = BM / 32;
  static constexpr int T = 64 * NW;
  static constexpr int QS = BF16 ? D / 16 : D / 2;  // MFMA k-steps over d
  static constexpr int OB = D / 32;                  // 32-wide d blocks of the output
  // LDS tiles [BN][KS] (K) and [BN][VS] (V), strides in elements.  bf16 V, and K at d = 64:
  // unpadded, chunks swizzled (vswz, kswz); bf16 K at d = 128: rows padded to 272 bytes (16
  // consecutive rows then start on 16 consecutive 16-byte bank groups, and the reads keep
  // immediate offsets); f32: padded rows
  static constexpr bool KPAD = !BF16 || D == 128;
  static constexpr int KS = BF16 ? (KPAD ? D + 8 : D) : D + 1;
  static constexpr int VS = BF16 ? D : D + 4;
  static constexpr int ROWB = BF16 ? 2 * D : 0;      // bytes per bf16 key row
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = BN * VS;
  // tile fetch: a task is 4 keys (bf16: kq + 16u, f32: 4 kq + u, u = 0..3) x one 16-byte chunk
  // of K and of V
  static constexpr int EPC = BF16 ? 8 : 4;            // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                 // chunks per key row
  static constexpr int TASKS = (BN / 4) * CPR;
  static constexpr int NT = (TASKS + T - 1) / T;      // tasks per thread
  using elem = typename std::conditional<BF16, unsigned short, float>::type;
};

// Work-item decode: blockIdx -> (batch, head, row block).  Workgroup k runs on XCD k % 8.
// When the row blocks split into 8 * kChunk-block pieces, the kv groups are taken one after
// another by all eight XCDs together (one group's K/V, 32 MiB at S = 64K and d = 128, is what the
// whole chip reads at a time), each XCD taking chunks of kChunk neighbouring row blocks (which
// share band tiles in its L2), chunks dealt round-robin, heaviest (last) row blocks first, and
// inside a chunk the row blocks of one head before the next head (measured 5 % faster at S = 64K
// than heads innermost).  Otherwise, when batch * hkv is a multiple of 8, each XCD owns
// whole kv groups; else plain descending row-block order.
constexpr int kChunk = 4;

__device__ inline void decode_item(const Params& p, int& b, int& h, int& rb) {
  const int k = blockIdx.x;
  const int G = p.B * p.hkv, hpg = p.hq / p.hkv;
  const int x = k & 7, s = k >> 3;
  if (p.nb % (8 * kChunk) == 0) {
    const int per_xcd_group = (p.nb / 8) * hpg;  // items of one kv group on one XCD
    const int g = s / per_xcd_group, r = s % per_xcd_group;
    const int cl = r / (kChunk * hpg), rr = r % (kChunk * hpg);
    const int c = p.nb / kChunk - 1 - (cl * 8 + x);
    rb = c * kChunk + (kChunk - 1 - rr % kChunk);
    b = g / p.hkv;
    h = (g % p.hkv) * hpg + rr / kChunk;
  } else if ((G & 7) == 0) {
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

// One key tile of a work item (wave-uniform): kind 1 = contiguous keys j0 .. j0+nvalid-1 of a
// segment, kind 2 = gathered columns col_idx[pc .. pc+nvalid), kind 0 = past the last tile.
struct Tile {
  int kind, j0, shi, nvalid;
  int64_t seg, pc;
};

template <bool REFILL>
struct TileWalk {
  int64_t s1, c0, c1;
  ListStream<2, REFILL> segs;  // seg_lo, seg_hi

  __device__ Tile first(int64_t s0) {
    Tile t;
    t.seg = s0;
    t.pc = c0;
    if (s0 < s1) {
      t.kind = 1;
      t.j0 = segs.get(0, s0);
      t.shi = segs.get(1, s0);
      t.nvalid = min(BN, t.shi - t.j0 + 1);
    } else {
      start_gather(t);
    }
    return t;
  }
  __device__ void start_gather(Tile& t) const {
    t.j0 = 0;
    t.shi = 0;
    if (c0 < c1) {
      t.kind = 2;
      t.pc = c0;
      t.nvalid = (int)min((int64_t)BN, c1 - c0);
    } else {
      t.kind = 0;
      t.nvalid = 0;
    }
  }
  __device__ Tile next(Tile t) {
    if (t.kind == 1) {
      if (t.j0 + BN <= t.shi) {
        t.j0 += BN;
      } else if (++t.seg < s1) {
        t.j0 = segs.get(0, t.seg);
        t.shi = segs.get(1, t.seg);
      } else {
        start_gather(t);
        return t;
      }
      t.nvalid = min(BN, t.shi - t.j0 + 1);
    } else if (t.kind == 2) {
      t.pc += BN;
      if (t.pc < c1) {
        t.nvalid = (int)min((int64_t)BN, c1 - t.pc);
      } else {
        t.kind = 0;
        t.nvalid = 0;
      }
    }
    return t;
  }
};

template <int D, int BM, bool BF16>
__global__ void __launch_bounds__(2 * BM) __attribute__((amdgpu_waves_per_eu(2))) k_attn(Params p) {  // 2*BM threads = BM/32 waves
  using C = Cfg<D, BM, BF16>;
  using E = typename C::elem;
  __shared__ __attribute__((aligned(16))) E Ks[C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) E Vs[C::V_ELEMS];
  __shared__ __attribute__((aligned(16))) int32_t cols_sh[3][BN];
  __shared__ int32_t list_sh[BM / 32][3 * 64];  // per wave: segment bounds, in-segment columns

  // the wave index is uniform: kept in a scalar register, so that row and LDS offsets derived from it
  // (and M0 of the LDS-direct loads) are scalar arithmetic
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  int b, h, rb;
  decode_item(p, b, h, rb);
  const int S = p.S;
  const int b0 = rb * BM, b1 = min(S, b0 + BM) - 1;
  const int i = b0 + wave * 32 + r32;  // this lane's query row
  // the item's list bounds, loaded together with Q (one round trip)
  const int64_t item = (int64_t)h * p.nb + rb;
  const int64_t lb_b0 = p.bcol_ptr[item], lb_b1 = p.bcol_ptr[item + 1], lb_s0 = p.seg_ptr[item],
                lb_s1 = p.seg_ptr[item + 1], lb_c0 = p.col_ptr[item], lb_c1 = p.col_ptr[item + 1];
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
  // Q is complete before the pipelined loop, so the loop's waits only ever cover the prefetch
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)

  f32x16 oacc[C::OB];
#pragma unroll
  for (int x = 0; x < C::OB; ++x)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[x][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // the first 64 segment bounds and in-segment columns of the item, loaded together
  TileWalk<false> walk;
  walk.s1 = uni64(lb_s1);
  walk.c0 = uni64(lb_c0);
  walk.c1 = uni64(lb_c1);
  walk.segs.src[0] = p.seg_lo;
  walk.segs.src[1] = p.seg_hi;
  walk.segs.sh = list_sh[wave];
  walk.segs.end = walk.s1;
  BcolStream<false> bcs;
  bcs.ls.src[0] = p.bcol_idx;
  bcs.ls.sh = list_sh[wave] + 128;
  bcs.ls.end = uni64(lb_b1);
  bcs.pos = uni64(lb_b0);
  const int64_t seg0 = uni64(lb_s0);
  walk.segs.issue(seg0);
  bcs.ls.issue(bcs.pos);
  walk.segs.commit();
  bcs.ls.commit();

  // ---- tile fetch: global -> registers (issued one tile ahead), registers -> LDS.
  // Buffer loads: an offset past the end of the kv head's slab reads as zero, so padding keys
  // (past nvalid, past S, threads without a task) need no branch.
  constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer, 32-bit data format
  const uint32_t slab_bytes = (uint32_t)S * D * sizeof(E);
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, slab_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, slab_bytes, kBufFlags);
  uint4 kreg[C::NT][4], vreg[C::NT][4];
  // key row of key u of task group kq: bf16 kq + 16u (the 16 lanes of one LDS write then cover
  // one 256-byte row, or two adjacent 128-byte rows), f32 4 kq + u
  auto krow = [](int kq, int u) { return BF16 ? kq + 16 * u : 4 * kq + u; };
  auto fetch = [&](const Tile& t, const int32_t* cols) {
#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
      const int x = tid + it * C::T;
      const int c = x % C::CPR, kq = x / C::CPR;
      const bool task = (C::TASKS % C::T == 0) || x < C::TASKS;
      int key[4];
      if (t.kind == 2 && task) {
        if constexpr (BF16) {
#pragma unroll
          for (int u = 0; u < 4; ++u) key[u] = cols[kq + 16 * u];
        } else {
          const int4 kc = *reinterpret_cast<const int4*>(&cols[4 * kq]);
          key[0] = kc.x;
          key[1] = kc.y;
          key[2] = kc.z;
          key[3] = kc.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = t.j0 + krow(kq, u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = task & (krow(kq, u) < t.nvalid) & (key[u] < S);
        const int off = ok ? key[u] * (D * (int)sizeof(E)) + 16 * c : (int)slab_bytes;
        auto kv = __builtin_amdgcn_raw_buffer_load_b128(rsK, off, 0, 0);
        auto vv = __builtin_amdgcn_raw_buffer_load_b128(rsV, off, 0, 0);
        kreg[it][u] = *reinterpret_cast<uint4*>(&kv);
        vreg[it][u] = *reinterpret_cast<uint4*>(&vv);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int it = 0; it < C::NT; ++it) {
      const int x = tid + it * C::T;
      if (x < C::TASKS) {
        const int c = x % C::CPR, kq = x / C::CPR;
        if constexpr (BF16) {
          // rows kq + 16u: the swizzles depend on the row mod 16 only, i.e. on kq
          unsigned char* Kb = reinterpret_cast<unsigned char*>(Ks);
          unsigned char* Vb = reinterpret_cast<unsigned char*>(Vs);
          constexpr int KROWB = 2 * C::KS;
          const int kp = kq * KROWB + 16 * (C::KPAD ? c : (c ^ kswz<D>(kq)));
          const int vp = kq * C::ROWB + 16 * (c ^ vswz<D>(kq));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            *reinterpret_cast<uint4*>(Kb + kp + 16 * u * KROWB) = kreg[it][u];
            *reinterpret_cast<uint4*>(Vb + vp + 16 * u * C::ROWB) = vreg[it][u];
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int kk = krow(kq, u);
            const float* kf = reinterpret_cast<const float*>(&kreg[it][u]);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ks[kk * C::KS + 4 * c + e] = kf[e];
            *reinterpret_cast<uint4*>(&Vs[kk * C::VS + 4 * c]) = vreg[it][u];
          }
        }
      }
    }
  };

  // ---- per-lane key mask of a tile, in two steps so that its loads overlap other work:
  // mask_loads issues the three diagonal-bitmap words that cover this lane's 64 offsets and
  // collects the tile's in-segment columns; mask_finish combines them with causality.
  const uint32_t* dbh = p.dbits + (int64_t)h * p.nwords;
  struct MaskIn {
    uint32_t w0, w1, w2;
    uint64_t xin;
  };
  auto mask_loads = [&](const Tile& t) -> MaskIn {
    MaskIn mi{0u, 0u, 0u, 0ull};
    if (t.kind == 1) {
      // offsets of keys j0 + 63 .. j0 of row i are base - 63 .. base (base = i - j0); the words
      // below offset 0 read as zero (out of the buffer)
      // (each word is loaded from a clamped index and zeroed when the index was out of range; the
      // three loads must stay separate, a merged wide buffer load would drop all three words when one
      // of them is out of range)
      const int wl = i - t.j0 - (BN - 1);
      const int wi = wl >> 5;
      const int c0 = min(max(wi, 0), p.nwords - 1), c1 = min(max(wi + 1, 0), p.nwords - 1),
                c2 = min(max(wi + 2, 0), p.nwords - 1);
      const uint32_t a0 = dbh[c0], a1 = dbh[c1], a2 = dbh[c2];
      mi.w0 = (c0 == wi) ? a0 : 0u;
      mi.w1 = (c1 == wi + 1) ? a1 : 0u;
      mi.w2 = (c2 == wi + 2) ? a2 : 0u;
      // in-segment columns of this tile (sorted list, consumed in tile order)
      mi.xin = bcs.take(t.j0, t.nvalid);
    }
    return mi;
  };
  auto mask_finish = [&](const Tile& t, const MaskIn& mi, const int32_t* cols) -> uint64_t {
    uint64_t m = 0;
    if (t.kind == 1) {
      const int base = i - t.j0;
      const int sh = (base - (BN - 1)) & 31;
      const uint64_t lo = ((uint64_t)mi.w1 << 32) | mi.w0;
      const uint64_t win = sh ? ((lo >> sh) | ((uint64_t)mi.w2 << (64 - sh))) : lo;
      // window bit q is offset base - 63 + q, i.e. key kk = 63 - q
      m = __builtin_bitreverse64(win) | mi.xin;
      m &= prefix_mask(t.nvalid) & prefix_mask(base + 1);
    } else if (t.kind == 2) {
      // gathered: the list is sorted, so the causal keys of row i are a prefix
      const int nvalid = t.nvalid;
      int cnt = nvalid;
      if (cols[nvalid - 1] > i) {
        int lo = 0, hi = nvalid;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (cols[mid] <= i) lo = mid + 1;
          else hi = mid;
        }
        cnt = lo;
      }
      m = prefix_mask(cnt);
    }
    return row_ok ? m : 0ull;
  };

  // per-lane LDS offsets of the bf16 operand reads.  K (swizzled rows), row r32, logical chunk
  // 2s + g: koff0 ^ 32s.  V, transposed read of d block x (key row 4 (q16 / 2) + es of each 16):
  // voff0 ^ 64x.  Both XORs stay inside the swizzled chunk bits of one row.
  int koff0 = 0, voff0 = 0;
  if constexpr (BF16) {
    koff0 = C::KPAD ? (r32 * C::KS + 8 * g) * 2 : r32 * C::ROWB + 16 * (g ^ kswz<D>(r32));
    const int q16 = lane >> 4, t16 = lane & 15, es = t16 >> 2, as = t16 & 3;
    const int d = 16 * (q16 & 1) + 4 * as;
    voff0 = (4 * (q16 >> 1) + es) * C::ROWB + 16 * ((d >> 3) ^ vswz<D>(es)) + 8 * ((d >> 2) & 1);
  }

  auto compute_tile = [&](uint64_t m) {
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
      if constexpr (BF16) {
#pragma unroll
        for (int s = 0; s < C::QS; ++s) {
          const int ko = C::KPAD ? kb * 32 * C::KS * 2 + koff0 + 32 * s : kb * 32 * C::ROWB + (koff0 ^ (32 * s));
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const unsigned char*>(Ks) + ko);
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
    // mask: value v of block kb is key kb*32 + 8*(v/4) + 4*g + v%4; the key's bit, sign-extended to a
    // whole word, keeps the score or inserts -inf (bit-field extract, bit-field insert)
    if (!__all(m == ~0ull)) {
      const uint64_t mg = m >> (4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t word = (uint32_t)(mg >> (32 * kb));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int bit = 8 * (v >> 2) + (v & 3);
          const uint32_t keep = (uint32_t)((int32_t)(word << (31 - bit)) >> 31);
          sacc[kb][v] = __uint_as_float((__float_as_uint(sacc[kb][v]) & keep) | (0xff800000u & ~keep));
        }
      }
    }
    // online softmax in the log2 domain.  The reference maximum moves only when the tile maximum
    // exceeds it by more than kLazy (probabilities up to 2^kLazy are exact enough in fp32 and keep
    // bf16's relative precision), so the O rescale is rare.
    constexpr float kLazy = 8.0f;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = pair_max(mx) * p.scale_log2;
    const bool move = mx > m_run + kLazy;
    if (__any(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < C::OB; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[x][v] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // bf16: one fma per score.  fp32: scale first, so a row maximum that sets the reference
        // maps to exp2(0) = 1 exactly.
        const float arg = BF16 ? __builtin_fmaf(sacc[kb][v], p.scale_log2, -m_use)
                               : mul_then_sub(sacc[kb][v], p.scale_log2, m_use);
        const float e = __builtin_amdgcn_exp2f(arg);
        sacc[kb][v] = e;
        if constexpr (!BF16) lsum += e;
      }
    if constexpr (!BF16) l_run += lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (BF16) {
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          bf16x8 pf;
#pragma unroll
          for (int t = 0; t < 8; ++t) pf[t] = (__bf16)sacc[kb][8 * mm + t];
          // the row sum of the same bf16 probabilities that weight V, two per instruction
          const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
          for (int t = 0; t < 8; t += 2)
            l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[t], pf[t + 1]}, ones, l_run, false);
          const unsigned char* Vb = reinterpret_cast<const unsigned char*>(Vs) + (kb * 32 + 16 * mm) * C::ROWB;
#pragma unroll
          for (int x = 0; x < C::OB; ++x) {
            const int vo = voff0 ^ (64 * x);
            const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vb + vo));
            const v4i16 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vb + 8 * C::ROWB + vo));
            const v8i16 vf = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf), pf, oacc[x], 0, 0, 0);
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

  // ---- software pipeline: the K/V tile and the mask inputs of tile t+1 and the column list of
  // tile t+2 are loaded while tile t is computed.  cols_sh[n % 3] holds the columns of gathered tile n.
  auto load_cols = [&](const Tile& t, int32_t* dst) {
    if (t.kind == 2 && tid < BN) dst[tid] = tid < t.nvalid ? p.col_idx[t.pc + tid] : 0;
  };
  Tile cur = walk.first(seg0);
  Tile nxt = walk.next(cur);
  Tile nn = walk.next(nxt);
  load_cols(cur, cols_sh[0]);
  load_cols(nxt, cols_sh[1]);
  __syncthreads();
  uint64_t m_cur = 0;
  if (cur.kind != 0) {
    const MaskIn mi = mask_loads(cur);
    fetch(cur, cols_sh[0]);
    m_cur = mask_finish(cur, mi, cols_sh[0]);
    store();
  }
  __syncthreads();
  for (int n = 0; cur.kind != 0; ++n) {
    const int bc = n % 3, bx = (n + 1) % 3, bz = (n + 2) % 3;
    (void)bc;
    MaskIn mi{0u, 0u, 0u, 0ull};
    if (nxt.kind != 0) {
      mi = mask_loads(nxt);
      fetch(nxt, cols_sh[bx]);
    }
    int32_t ncol = 0;
    if (nn.kind == 2 && tid < BN && tid < nn.nvalid) ncol = p.col_idx[nn.pc + tid];
    compute_tile(m_cur);
    const uint64_t m_next = nxt.kind != 0 ? mask_finish(nxt, mi, cols_sh[bx]) : 0ull;
    __syncthreads();
    if (nxt.kind != 0) store();
    if (nn.kind == 2 && tid < BN) cols_sh[bz][tid] = ncol;
    __syncthreads();
    m_cur = m_next;
    cur = nxt;
    nxt = nn;
    nn = walk.next(nn);
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

// ============================================================================
// bf16 kernel for 128-row blocks.  Four waves per workgroup: wave w owns rows
// 32w..32w+31 and all 64 keys of a tile, so four waves share every K/V tile.
// K and V tiles travel global -> LDS with buffer_load ... lds (no register
// staging), double-buffered: the loads of tile t+1 are in flight while tile t is
// computed, one barrier per tile.  Tiles are stored key-row-major with the
// 16-byte chunks of row R XOR-swizzled (K: chunk ^ kswz(R); V: chunk ^ 2(R % 4))
// (see kswz and vswz).  The V operand of O^T = V^T P^T is read with ds_read_b64_tr_b16, which transposes 4x4 blocks of
// 16-bit values across each group of 16 lanes: source lane a + 4e supplies 4
// consecutive d values of key row key0 + e, and lane 4a + b receives column b of
// those rows, i.e. 4 consecutive keys of one d -- the layout the MFMA A operand
// needs.  Row sums come from v_dot2_f32_bf16 on the packed probabilities.
// ============================================================================
template <int D, int BM>
struct Cfg3 {
  static constexpr int NW = BM / 32;
  static constexpr int T = 64 * NW;
  static constexpr int NKB = BN / 32;                 // 32-key blocks per tile
  static constexpr int QS = D / 16;
  static constexpr int OB = D / 32;
  static constexpr int ROWB = D * 2;                  // bytes per key row
  static constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  static constexpr int RPL = 64 / CPR;                // key rows per 1 KB load instruction
  static constexpr int LPW = (BN / RPL) / NW;         // load instructions per wave per matrix
  static constexpr int MAT = BN * ROWB;               // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * MAT;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

template <int D, int BM>
__global__ void __launch_bounds__(64 * (BM / 32)) __attribute__((amdgpu_waves_per_eu(2)))
k_attn_bf16(Params p) {
  using C = Cfg3<D, BM>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) int32_t cols_sh[3][BN];
  __shared__ int32_t list_sh[BM / 32][3 * 64];  // per wave: segment bounds, in-segment columns

  // the wave index is uniform: kept in a scalar register, so that row and LDS offsets derived from it
  // (and M0 of the LDS-direct loads) are scalar arithmetic
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  const int rh = wave;  // this wave's 32 rows
  int b, h, rb;
  decode_item(p, b, h, rb);
  const int S = p.S;
  const int b0 = rb * BM, b1 = min(S, b0 + BM) - 1;
  const int i = b0 + rh * 32 + r32;
  // the item's list bounds, loaded together with Q (one round trip)
  const int64_t item = (int64_t)h * p.nb + rb;
  const int64_t lb_b0 = p.bcol_ptr[item], lb_b1 = p.bcol_ptr[item + 1], lb_s0 = p.seg_ptr[item],
                lb_s1 = p.seg_ptr[item + 1], lb_c0 = p.col_ptr[item], lb_c1 = p.col_ptr[item + 1];
  const bool row_ok = i <= b1;
  const int kvh = h / (p.hq / p.hkv);
  using E = unsigned short;
  const E* Qg = static_cast<const E*>(p.q) + ((int64_t)(b * p.hq + h) * S) * D;
  const E* Kg = static_cast<const E*>(p.k) + ((int64_t)(b * p.hkv + kvh) * S) * D;
  const E* Vg = static_cast<const E*>(p.v) + ((int64_t)(b * p.hkv + kvh) * S) * D;

  bf16x8 qf[C::QS];
#pragma unroll
  for (int s = 0; s < C::QS; ++s) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (row_ok) u = *reinterpret_cast<const uint4*>(Qg + (int64_t)i * D + 16 * s + 8 * g);
    qf[s] = *reinterpret_cast<bf16x8*>(&u);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): Q is in registers before the pipelined loop

  f32x16 oacc[C::OB];
#pragma unroll
  for (int x = 0; x < C::OB; ++x)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[x][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // the first 64 segment bounds and in-segment columns of the item, loaded together
  TileWalk<true> walk;
  walk.s1 = uni64(lb_s1);
  walk.c0 = uni64(lb_c0);
  walk.c1 = uni64(lb_c1);
  walk.segs.src[0] = p.seg_lo;
  walk.segs.src[1] = p.seg_hi;
  walk.segs.sh = list_sh[wave];
  walk.segs.end = walk.s1;
  BcolStream<true> bcs;
  bcs.ls.src[0] = p.bcol_idx;
  bcs.ls.sh = list_sh[wave] + 128;
  bcs.ls.end = uni64(lb_b1);
  bcs.pos = uni64(lb_b0);
  const int64_t seg0 = uni64(lb_s0);
  walk.segs.issue(seg0);
  bcs.ls.issue(bcs.pos);
  walk.segs.commit();
  bcs.ls.commit();

  constexpr uint32_t kBufFlags = 0x00020000u;
  const uint32_t slab_bytes = (uint32_t)S * D * 2u;
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc((void*)Kg, 0, slab_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rsV = __builtin_amdgcn_make_buffer_rsrc((void*)Vg, 0, slab_bytes, kBufFlags);

  // ---- tile loads straight into LDS stage `st`: wave w fills key rows [w*LPW*RPL, (w+1)*LPW*RPL)
  // lane constants of the tile loads: key row R = R0 + lane / CPR, chunk slot P = lane % CPR.
  // R0 is a multiple of RPL (4 or 8) and the wave's first row a multiple of 16, so
  // kswz(R) = kswz(k * RPL) ^ kswz(lane / CPR), and R % 4 == (lane / CPR) % 4.
  const int ld_r = lane / C::CPR, ld_p = lane % C::CPR;
  static_assert((C::LPW * C::RPL) % 16 == 0, "each wave's first tile row must be a multiple of 16");
  const int ld_ck = 16 * (ld_p ^ kswz<D>(ld_r)), ld_cv = 16 * (ld_p ^ vswz<D>(ld_r)), ld_row = ld_r * C::ROWB;
  auto issue_tile = [&](const Tile& t, int st, const int32_t* cols) __attribute__((always_inline)) {
    unsigned char* Kst = lds + st * C::STAGE;
    unsigned char* Vst = Kst + C::MAT;
    int key[C::LPW];
#pragma unroll
    for (int k = 0; k < C::LPW; ++k) key[k] = t.j0 + (wave * C::LPW + k) * C::RPL + ld_r;
    if (t.kind == 2) {
#pragma unroll
      for (int k = 0; k < C::LPW; ++k) key[k] = cols[(wave * C::LPW + k) * C::RPL + ld_r];
    }
    // rows of the tile that hold keys (< S for a band tile; list entries are always < S)
    const int lim = t.kind == 2 ? t.nvalid : min(t.nvalid, S - t.j0);
    if (lim == BN && t.kind == 1) {
      // whole band tile: the row offset is uniform (scalar offset), the lane part a constant
#pragma unroll
      for (int k = 0; k < C::LPW; ++k) {
        const int R0 = (wave * C::LPW + k) * C::RPL;
        const int so = (t.j0 + R0) * C::ROWB;
        const int ck = ld_ck ^ (16 * kswz<D>(k * C::RPL));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_void_ptr)(Kst + R0 * C::ROWB), 16, ld_row + ck, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_void_ptr)(Vst + R0 * C::ROWB), 16, ld_row + ld_cv, so, 0, 0);
      }
    } else if (lim == BN) {
      // whole gathered tile: every row holds a key
#pragma unroll
      for (int k = 0; k < C::LPW; ++k) {
        const int R0 = (wave * C::LPW + k) * C::RPL;
        const int base = key[k] * C::ROWB;
        const int ck = ld_ck ^ (16 * kswz<D>(k * C::RPL));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_void_ptr)(Kst + R0 * C::ROWB), 16, base + ck, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_void_ptr)(Vst + R0 * C::ROWB), 16, base + ld_cv, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::LPW; ++k) {
        const int R0 = (wave * C::LPW + k) * C::RPL;
        const int base = R0 + ld_r < lim ? key[k] * C::ROWB : (int)slab_bytes;  // past the slab: zeros
        const int ck = ld_ck ^ (16 * kswz<D>(k * C::RPL));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (lds_void_ptr)(Kst + R0 * C::ROWB), 16, base + ck, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (lds_void_ptr)(Vst + R0 * C::ROWB), 16, base + ld_cv, 0, 0, 0);
      }
    }
  };

  // ---- per-lane 64-bit key mask of a tile (see the fp32 kernel for the derivation)
  const uint32_t* dbh = p.dbits + (int64_t)h * p.nwords;
  struct MaskIn {
    uint32_t w0, w1, w2;
    uint64_t xin;
    bool full;  // every key of the tile is retained for every row of the block (wave-uniform)
    bool cand;  // band tile that may be full: decided in mask_finish from fw
    uint32_t fw;
  };
  // the offsets a band tile shows the block, [b0 - j0 - 63, b1 - j0], span at most BM + 63 bits,
  // i.e. at most kWords bitmap words from word omin / 32; lane k < kWords holds word k of them
  constexpr int kWords = (BM + BN - 1 + 31) / 32 + 1;
  auto mask_loads = [&](const Tile& t, const int32_t* cols) __attribute__((always_inline)) -> MaskIn {
    MaskIn mi{0u, 0u, 0u, 0ull, false, false, 0u};
    if (t.kind == 2) mi.full = (t.nvalid == BN) && (cols[BN - 1] <= b0);
    if (t.kind == 1) {
      // full when the whole tile is at or below the block's first row and every offset any row of
      // the block sees in it is a diagonal: one vector load spreads the words over lanes, and
      // mask_finish checks them (by then the load has had the current tile's compute to land)
      if (t.nvalid == BN && t.j0 + BN - 1 <= b0) {
        const int w = ((b0 - t.j0 - (BN - 1)) >> 5) + min(lane, kWords - 1);
        mi.cand = true;
        mi.fw = dbh[min(w, p.nwords - 1)];
      }
      const int wl = i - t.j0 - (BN - 1);
      const int wi = wl >> 5;
      const int c0 = min(max(wi, 0), p.nwords - 1), c1 = min(max(wi + 1, 0), p.nwords - 1),
                c2 = min(max(wi + 2, 0), p.nwords - 1);
      const uint32_t a0 = dbh[c0], a1 = dbh[c1], a2 = dbh[c2];
      mi.w0 = (c0 == wi) ? a0 : 0u;
      mi.w1 = (c1 == wi + 1) ? a1 : 0u;
      mi.w2 = (c2 == wi + 2) ? a2 : 0u;
      mi.xin = bcs.take(t.j0, t.nvalid);
    }
    return mi;
  };
  auto mask_finish = [&](const Tile& t, const MaskIn& mi, const int32_t* cols) __attribute__((always_inline)) -> uint64_t {
    if (mi.full) return ~0ull;
    if (mi.cand) {
      const int omin = b0 - t.j0 - (BN - 1), omax = b1 - t.j0;
      const int w = (omin >> 5) + lane;
      const int a = max(omin - 32 * w, 0), e = min(omax - 32 * w, 31);
      const uint32_t need =
          (lane < kWords && a <= e) ? ((e == 31 ? 0xffffffffu : ((1u << (e + 1)) - 1u)) & ~((1u << a) - 1u)) : 0u;
      if (__all((mi.fw & need) == need)) return ~0ull;
    }
    uint64_t m = 0;
    if (t.kind == 1) {
      const int base = i - t.j0;
      const int sh = (base - (BN - 1)) & 31;
      const uint64_t lo = ((uint64_t)mi.w1 << 32) | mi.w0;
      const uint64_t win = sh ? ((lo >> sh) | ((uint64_t)mi.w2 << (64 - sh))) : lo;
      m = __builtin_bitreverse64(win) | mi.xin;
      m &= prefix_mask(t.nvalid) & prefix_mask(base + 1);
    } else if (t.kind == 2) {
      const int nvalid = t.nvalid;
      int cnt = nvalid;
      if (cols[nvalid - 1] > i) {
        int lo = 0, hi = nvalid;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (cols[mid] <= i) lo = mid + 1;
          else hi = mid;
        }
        cnt = lo;
      }
      m = prefix_mask(cnt);
    }
    return row_ok ? m : 0ull;
  };

  // per-lane LDS offsets that do not change from tile to tile
  int koff[4];  // K row r32, logical chunk 2s + g for s = 0..3 (s + 4: chunk + 8, offset ^ 128)
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = r32 * C::ROWB + 16 * ((2 * s + g) ^ kswz<D>(r32));
  const int q16 = lane >> 4, t16 = lane & 15, es = t16 >> 2, as = t16 & 3;
  int voff[C::OB];  // transposed-read source address for d block x (key row key0 + es)
#pragma unroll
  for (int x = 0; x < C::OB; ++x) {
    const int d = 32 * x + 16 * (q16 & 1) + 4 * as;
    voff[x] = (4 * (q16 >> 1) + es) * C::ROWB + 16 * ((d >> 3) ^ vswz<D>(es)) + 8 * ((d >> 2) & 1);
  }

  auto compute_tile = [&](int st, uint64_t m) __attribute__((always_inline)) {
    const unsigned char* Kst = lds + st * C::STAGE;
    const unsigned char* Vst = Kst + C::MAT;
    f32x16 sacc[C::NKB];
    // all K fragments of the tile first, so that the MFMA burst below waits for LDS only once
    bf16x8 kf[C::NKB][C::QS];
#pragma unroll
    for (int kbl = 0; kbl < C::NKB; ++kbl)
#pragma unroll
      for (int s = 0; s < C::QS; ++s)
        kf[kbl][s] = *reinterpret_cast<const bf16x8*>(Kst + kbl * 32 * C::ROWB + (koff[s & 3] ^ ((s >> 2) * 128)));
#pragma unroll
    for (int kbl = 0; kbl < C::NKB; ++kbl) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kbl][v] = 0.0f;
#pragma unroll
      for (int s = 0; s < C::QS; ++s)
        sacc[kbl] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kbl][s], qf[s], sacc[kbl], 0, 0, 0);
    }
    // all V fragments (transposed reads) next; they do not depend on the softmax and their
    // latency hides behind it
    v8i16 vfr[C::NKB][2][C::OB];
#pragma unroll
    for (int kbl = 0; kbl < C::NKB; ++kbl)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int kbase = (kbl * 32 + 16 * mm) * C::ROWB;
#pragma unroll
        for (int x = 0; x < C::OB; ++x) {
          const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vst + kbase + voff[x]));
          const v4i16 vb =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(Vst + kbase + 8 * C::ROWB + voff[x]));
          vfr[kbl][mm][x] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    // mask: value v of block kbl is key kbl*32 + 8*(v/4) + 4*g + v%4.  Per value, the key's bit is
    // sign-extended into an all-ones / all-zeros word, which keeps the score or inserts -inf (two
    // instructions: bit-field extract, bit-field insert).
    const uint64_t mw = m >> (4 * g);
    if (!__all(m == ~0ull)) {
#pragma unroll
      for (int kbl = 0; kbl < C::NKB; ++kbl) {
        const uint32_t word = (uint32_t)(mw >> (32 * kbl));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int bit = 8 * (v >> 2) + (v & 3);
          const uint32_t keep = (uint32_t)((int32_t)(word << (31 - bit)) >> 31);
          sacc[kbl][v] = __uint_as_float((__float_as_uint(sacc[kbl][v]) & keep) | (0xff800000u & ~keep));
        }
      }
    }
    constexpr float kLazy = 8.0f;
    float mx = -INFINITY;
#pragma unroll
    for (int kbl = 0; kbl < C::NKB; ++kbl)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kbl][v]);
    mx = pair_max(mx) * p.scale_log2;
    const bool move = mx > m_run + kLazy;
    if (__any(move)) {
      const float m_new = move ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < C::OB; ++x)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[x][v] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kbl = 0; kbl < C::NKB; ++kbl) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        bf16x8 pf;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          pf[t] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbl][8 * mm + t], p.scale_log2, -m_use));
#pragma unroll
        for (int t = 0; t < 8; t += 2) l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[t], pf[t + 1]}, ones, l_run, false);
#pragma unroll
        for (int x = 0; x < C::OB; ++x)
          oacc[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vfr[kbl][mm][x]), pf, oacc[x],
                                                            0, 0, 0);
      }
    }
  };

  // ---- pipeline
  auto load_cols = [&](const Tile& t, int32_t* dst) {
    if (t.kind == 2 && tid < BN) dst[tid] = tid < t.nvalid ? p.col_idx[t.pc + tid] : 0;
  };
  Tile cur = walk.first(seg0);
  Tile nxt = walk.next(cur);
  Tile nn = walk.next(nxt);
  load_cols(cur, cols_sh[0]);
  load_cols(nxt, cols_sh[1]);
  __syncthreads();
  uint64_t m_cur = 0;
  if (cur.kind != 0) {
    const MaskIn mi = mask_loads(cur, cols_sh[0]);
    issue_tile(cur, 0, cols_sh[0]);
    m_cur = mask_finish(cur, mi, cols_sh[0]);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // this thread's tile loads have landed in LDS
  __syncthreads();
  // one tile step; the LDS stage of tile n is n & 1, passed as a constant (the loop below takes two
  // steps per iteration), so the stage offsets of the tile's reads fold into the LDS instructions'
  // immediate offsets.  The next tile's loads take the stage as a run-time value: their LDS bases (M0)
  // are then computed per tile instead of being held for both stages, which would spill SGPRs.
  auto tile_step = [&](int n, auto stage) __attribute__((always_inline)) {
    constexpr int st = decltype(stage)::value;
    const int bx = (n + 1) % 3, bz = (n + 2) % 3;
    MaskIn mi{0u, 0u, 0u, 0ull, false, false, 0u};
    if (nxt.kind != 0) {
      mi = mask_loads(nxt, cols_sh[bx]);
      int ld_stage = st ^ 1;
      asm volatile("" : "+s"(ld_stage));  // opaque to the optimizer: no constant to hoist per stage
      issue_tile(nxt, ld_stage, cols_sh[bx]);
    }
    int32_t ncol = 0;
    if (nn.kind == 2 && tid < BN && tid < nn.nvalid) ncol = p.col_idx[nn.pc + tid];
    compute_tile(st, m_cur);
    const uint64_t m_next = nxt.kind != 0 ? mask_finish(nxt, mi, cols_sh[bx]) : 0ull;
    if (nn.kind == 2 && tid < BN) cols_sh[bz][tid] = ncol;
    __builtin_amdgcn_s_waitcnt(0xF70);
    __syncthreads();
    m_cur = m_next;
    cur = nxt;
    nxt = nn;
    nn = walk.next(nn);
  };
  for (int n = 0; cur.kind != 0; n += 2) {
    tile_step(n, std::integral_constant<int, 0>{});
    if (cur.kind == 0) break;
    tile_step(n + 1, std::integral_constant<int, 1>{});
  }

  // ---- normalise and store
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
    E* Og = static_cast<E*>(p.o) + ((int64_t)(b * p.hq + h) * S + i) * D;
#pragma unroll
    for (int x = 0; x < C::OB; ++x)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * x + 8 * qd + 4 * g;
        __bf16 t4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = (__bf16)(oacc[x][4 * qd + e] * inv);
        *reinterpret_cast<uint2*>(Og + d0) = *reinterpret_cast<uint2*>(t4);
      }
    if (p.lse != nullptr && g == 0) {
      p.lse[(int64_t)(b * p.hq + h) * S + i] =
          l_tot > 0.0f ? m_run * 0.69314718055994530942f + logf(l_tot) : -INFINITY;
    }
  }
}

template <int D, int BM>
hipError_t launch_bf16(const Params& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.B * p.hq * p.nb;
  k_attn_bf16<D, BM><<<dim3((unsigned)blocks), dim3(Cfg3<D, BM>::T), 0, stream>>>(p);
  return hipGetLastError();
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
  p.dbits = a.idx->dbits;
  p.nwords = ((a.S - 1) >> 5) + 1;
  // bf16: 128-row blocks run the LDS-direct kernel; 64-row blocks (two waves per block) run the
  // register-staged kernel, which keeps four blocks per CU and measured faster at that size.
  if (a.dtype == SA_DTYPE_BF16) {
    if (p.BM == 128) return a.head_dim == 64 ? launch_bf16<64, 128>(p, stream) : launch_bf16<128, 128>(p, stream);
    return a.head_dim == 64 ? launch_t<64, 64, true>(p, stream) : launch_t<128, 64, true>(p, stream);
  }
  return a.head_dim == 64 ? launch_bm<64, false>(p, stream) : launch_bm<128, false>(p, stream);
}

}  // namespace sa
