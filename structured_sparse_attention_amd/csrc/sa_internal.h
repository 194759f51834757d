// sa_internal.h -- declarations shared by the host entry points and the kernel files of libsa.so.
#pragma once

#include <hip/hip_runtime.h>

#include "sa.h"

namespace sa {

// Largest sequence length the index builder accepts: two bitmaps of S bits live in LDS.
constexpr int32_t kMaxIndexS = 262144;
// Largest capture window (two int32 hit arrays of L entries live in LDS).
constexpr int32_t kMaxCaptureL = 4096;
constexpr int32_t kMaxSampleRows = 2048;       // sampled rows per call
constexpr int64_t kMaxSampleRowSeqs = 1 << 20; // batch * rows per call: fixed-point totals < 2^52

// Index builder (sa_index.hip).  All launches go on `stream`.  Order of a build: heads, items (count),
// scan, [size query], items (fill), heads (fill).
hipError_t launch_index_heads(const sa_pattern_desc& d, const sa_index& ix, int32_t validate, hipStream_t stream);
hipError_t launch_index_items(const sa_pattern_desc& d, const sa_index& ix, int32_t fill, int32_t validate,
                              hipStream_t stream);
hipError_t launch_index_scan(const sa_index& ix, hipStream_t stream);
hipError_t launch_index_heads_fill(const sa_pattern_desc& d, const sa_index& ix, hipStream_t stream);

// Attention (sa_attn.hip).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t batch, hq, hkv, S, head_dim, dtype;
  float scale;
  const sa_index* idx;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

// Decode (sa_decode.hip): one query row per sequence at position pos[b].
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* pos;
  void* o;
  float* lse;
  int32_t batch, hq, hkv, S, head_dim, dtype;
  float scale;
  const sa_index* idx;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Pattern capture and extension (sa_capture.hip).
hipError_t launch_capture(const float* maps, int32_t n_maps, int32_t L, double lambda, double eps, double tau,
                          double mu, int32_t norm_scope, uint8_t* keep_diag, uint8_t* keep_vert, int32_t* diag_hits,
                          int32_t* vert_hits, uint8_t* true_mask, hipStream_t stream);
hipError_t launch_attention_maps(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t L,
                                 int32_t head_dim, int32_t dtype, float scale, float* maps, hipStream_t stream);
size_t sample_workspace_bytes(int32_t batch, int32_t hq, int32_t row0, int32_t n_rows);
// Static scratch of the allocation-free sample-scores entry point (one per GPU), and its device
// address on the current device (looked up once per device).
constexpr size_t kSampleStaticScratchBytes = (size_t)16 << 20;
hipError_t sample_static_scratch(void** out);
hipError_t launch_sample_scores(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                                int32_t head_dim, int32_t dtype, float scale, int32_t row0, int32_t n_rows,
                                int32_t band, const uint8_t* skip_cols, bool lse_given, float* row_lse, void* workspace,
                                int64_t* diag, int64_t* vert, hipStream_t stream);
hipError_t launch_select(const int64_t* scores, int32_t n_heads, int32_t S, double alpha, int64_t t_all, int32_t band,
                         uint8_t* keep, hipStream_t stream);
hipError_t launch_calib_mfma(int32_t n_wg, int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_calib_gather(const void* buf, int64_t region_bytes, int32_t chunk_bytes, int32_t n_wg, int32_t reads,
                               uint64_t seed, float* sink, hipStream_t stream);
hipError_t launch_coverage(const float* maps, int32_t n_maps, int32_t L, const uint8_t* keep_diag,
                           const uint8_t* keep_vert, double* mass, int64_t* cells, hipStream_t stream);
hipError_t launch_patterns_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L,
                                   int32_t S, int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr,
                                   int32_t* vert_col, hipStream_t stream);

}  // namespace sa
