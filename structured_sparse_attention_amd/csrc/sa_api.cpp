// sa_api.cpp -- C ABI entry points of libsa.so: host-side validation, then launches.
// Every check below runs before anything is enqueued, so an error return other
// than SA_ERR_HIP means no device work was started.
#include <math.h>

#include "sa_internal.h"

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

sa_status hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }
// element rows are moved in 16-byte vectors
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool index_arrays_ok(const sa_index& ix) {
  return ix.run_ptr && ix.run_lo && ix.run_hi && ix.seg_ptr && ix.seg_lo && ix.seg_hi && ix.bcol_ptr &&
         ix.bcol_idx && ix.col_ptr && ix.col_idx && ix.dbits;
}

}  // namespace

extern "C" {

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_DESC_INVALID: return "pattern descriptor is not sorted, unique and in range";
    case SA_ERR_CAPACITY: return "output capacity too small";
    case SA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sa_version(void) { return "libsa 0.1.0 gfx950"; }

sa_status sa_build_index(const sa_pattern_desc* desc, sa_index* idx, sa_index_sizes* sizes, int32_t flags,
                         void* stream) {
  if (desc == nullptr || idx == nullptr) return SA_ERR_INVALID_ARG;
  const sa_pattern_desc& d = *desc;
  if (d.S < 1 || d.n_heads < 1) return SA_ERR_INVALID_ARG;
  if (!d.diag_ptr || !d.diag_off || !d.vert_ptr || !d.vert_col) return SA_ERR_INVALID_ARG;
  if (idx->S != d.S || idx->n_heads != d.n_heads) return SA_ERR_INVALID_ARG;
  const int32_t BM = idx->row_block;
  if (BM != 64 && BM != 128) return SA_ERR_INVALID_ARG;
  if (idx->n_row_blocks != cdiv(d.S, BM)) return SA_ERR_INVALID_ARG;
  if (d.block_mask && (d.block_size < BM || d.block_size % BM != 0)) return SA_ERR_INVALID_ARG;
  if (d.stripe_ptr && (!d.stripe_col || d.stripe_rows < BM || d.stripe_rows % BM != 0)) return SA_ERR_INVALID_ARG;
  if (!idx->run_ptr || !idx->seg_ptr || !idx->bcol_ptr || !idx->col_ptr || !idx->pair_count || !idx->dbits ||
      !idx->status)
    return SA_ERR_INVALID_ARG;
  if ((int64_t)d.n_heads * idx->n_row_blocks > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
  if (d.S > sa::kMaxIndexS) return SA_ERR_UNSUPPORTED;
  const bool payload = idx->run_lo && idx->run_hi && idx->seg_lo && idx->seg_hi && idx->bcol_idx && idx->col_idx;
  if (!payload && sizes == nullptr) return SA_ERR_INVALID_ARG;
  if (payload && (idx->capacity.n_runs < 0 || idx->capacity.n_segs < 0 || idx->capacity.n_bcols < 0 ||
                  idx->capacity.n_cols < 0))
    return SA_ERR_INVALID_ARG;
  const int32_t validate = (flags & SA_BUILD_VALIDATE) ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);

  sa_index ix = *idx;
  if (!payload) {
    ix.run_lo = ix.run_hi = ix.seg_lo = ix.seg_hi = ix.bcol_idx = ix.col_idx = nullptr;
  }
  hipError_t e = sa::launch_index_heads(d, ix, validate, st);
  if (e == hipSuccess) e = sa::launch_index_items(d, ix, 0, validate, st);
  if (e == hipSuccess) e = sa::launch_index_scan(ix, st);
  if (e != hipSuccess) return SA_ERR_HIP;

  if (sizes != nullptr) {
    const int64_t n = (int64_t)d.n_heads * ix.n_row_blocks;
    int32_t nr = 0, status = 0;
    int64_t ns = 0, nbc = 0, nc = 0;
    e = hipMemcpyAsync(&nr, ix.run_ptr + d.n_heads, sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(&ns, ix.seg_ptr + n, sizeof(int64_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(&nbc, ix.bcol_ptr + n, sizeof(int64_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(&nc, ix.col_ptr + n, sizeof(int64_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(&status, ix.status, sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return SA_ERR_HIP;
    sizes->n_runs = nr;
    sizes->n_segs = ns;
    sizes->n_bcols = nbc;
    sizes->n_cols = nc;
    if (status & SA_STATUS_DESC_INVALID) return SA_ERR_DESC_INVALID;
    if (payload && (nr > idx->capacity.n_runs || ns > idx->capacity.n_segs || nbc > idx->capacity.n_bcols ||
                    nc > idx->capacity.n_cols))
      return SA_ERR_CAPACITY;
  }
  if (!payload) return SA_OK;
  e = sa::launch_index_items(d, ix, 1, 0, st);
  if (e == hipSuccess) e = sa::launch_index_heads_fill(d, ix, st);
  return hip_status(e);
}

size_t sa_build_index_workspace_bytes(const sa_pattern_desc* desc, int32_t row_block) {
  (void)desc;
  (void)row_block;
  return 0;  // counts and kinds live in the index's own arrays; the scans run in place
}

sa_status sa_sparse_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int32_t batch,
                                 int32_t hq, int32_t hkv, int32_t S, int32_t head_dim, int32_t dtype,
                                 float softmax_scale, const sa_index* idx, void* stream) {
  if (!q || !k || !v || !o || !idx) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SA_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || S < 1 || hq % hkv != 0) return SA_ERR_INVALID_ARG;
  if (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32) return SA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (idx->S != S || idx->n_heads != hq) return SA_ERR_INVALID_ARG;
  if ((idx->row_block != 64 && idx->row_block != 128) || idx->n_row_blocks != cdiv(S, idx->row_block))
    return SA_ERR_INVALID_ARG;
  if (!index_arrays_ok(*idx)) return SA_ERR_INVALID_ARG;
  if ((int64_t)batch * hq * idx->n_row_blocks > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  if (!isfinite(scale)) return SA_ERR_INVALID_ARG;
  sa::AttnArgs a{q, k, v, o, lse, batch, hq, hkv, S, head_dim, dtype, scale, idx};
  return hip_status(sa::launch_attention(a, static_cast<hipStream_t>(stream)));
}

sa_status sa_sparse_attn_decode(const void* q, const void* k, const void* v, const int32_t* pos, void* o, float* lse,
                                int32_t batch, int32_t hq, int32_t hkv, int32_t S, int32_t head_dim, int32_t dtype,
                                float softmax_scale, const sa_index* idx, void* stream) {
  if (!q || !k || !v || !pos || !o || !idx) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SA_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || S < 1 || hq % hkv != 0) return SA_ERR_INVALID_ARG;
  if (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32) return SA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (idx->S != S || idx->n_heads != hq) return SA_ERR_INVALID_ARG;
  if ((idx->row_block != 64 && idx->row_block != 128) || idx->n_row_blocks != cdiv(S, idx->row_block))
    return SA_ERR_INVALID_ARG;
  if (!index_arrays_ok(*idx)) return SA_ERR_INVALID_ARG;
  if ((int64_t)batch * hq > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  if (!isfinite(scale)) return SA_ERR_INVALID_ARG;
  sa::DecodeArgs a{q, k, v, pos, o, lse, batch, hq, hkv, S, head_dim, dtype, scale, idx};
  return hip_status(sa::launch_decode(a, static_cast<hipStream_t>(stream)));
}

sa_status sa_pattern_capture(const float* maps, int32_t n_maps, int32_t L, double lambda, double eps, double tau,
                             double mu, int32_t norm_scope, uint8_t* keep_diag, uint8_t* keep_vert,
                             int32_t* diag_hits, int32_t* vert_hits, uint8_t* true_mask, void* stream) {
  if (!maps || !keep_diag || !keep_vert) return SA_ERR_INVALID_ARG;
  if (n_maps < 1 || L < 1) return SA_ERR_INVALID_ARG;
  if (norm_scope != 0 && norm_scope != 1) return SA_ERR_INVALID_ARG;
  if (!isfinite(eps) || !isfinite(tau) || !isfinite(mu) || !isfinite(lambda)) return SA_ERR_INVALID_ARG;
  if (lambda <= 0.0 && !(eps > 0.0)) return SA_ERR_INVALID_ARG;  // A = 0 would give an infinite transform
  if (L > sa::kMaxCaptureL) return SA_ERR_UNSUPPORTED;
  return hip_status(sa::launch_capture(maps, n_maps, L, lambda, eps, tau, mu, norm_scope, keep_diag, keep_vert,
                                       diag_hits, vert_hits, true_mask, static_cast<hipStream_t>(stream)));
}

sa_status sa_pattern_coverage(const float* maps, int32_t n_maps, int32_t L, const uint8_t* keep_diag,
                              const uint8_t* keep_vert, double* mass, int64_t* cells, void* stream) {
  if (!maps || !keep_diag || !keep_vert || !mass) return SA_ERR_INVALID_ARG;
  if (n_maps < 1 || L < 1) return SA_ERR_INVALID_ARG;
  if (L > sa::kMaxCaptureL) return SA_ERR_UNSUPPORTED;
  return hip_status(sa::launch_coverage(maps, n_maps, L, keep_diag, keep_vert, mass, cells,
                                        static_cast<hipStream_t>(stream)));
}

size_t sa_sample_scores_workspace(int32_t batch, int32_t hq, int32_t row0, int32_t n_rows) {
  if (batch < 1 || hq < 1 || row0 < 0 || n_rows < 1) return 0;
  return sa::sample_workspace_bytes(batch, hq, row0, n_rows);
}

}  // extern "C"

namespace {

// Checks shared by the two sample-scores entry points (everything but the workspace).
sa_status sample_args_ok(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                         int32_t head_dim, int32_t dtype, float softmax_scale, int32_t row0, int32_t n_rows,
                         int32_t band, const float* row_lse, const int64_t* diag_score, const int64_t* vert_score,
                         float* scale_out) {
  if (!q || !k || !row_lse || (!diag_score && !vert_score)) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return SA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(diag_score) | reinterpret_cast<uintptr_t>(vert_score)) & 7u) return SA_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || S < 1 || hq % hkv != 0 || band < 0) return SA_ERR_INVALID_ARG;
  if (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32) return SA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (row0 < 0 || n_rows < 1 || (int64_t)row0 + n_rows > S) return SA_ERR_INVALID_ARG;
  if (n_rows > sa::kMaxSampleRows || (int64_t)batch * n_rows > sa::kMaxSampleRowSeqs) return SA_ERR_UNSUPPORTED;
  const int64_t ntile = ((int64_t)row0 + n_rows - 1) / 64 + 1;
  const int64_t nsplit = ((int64_t)row0 + n_rows - 1) / 256 + 1;
  if ((int64_t)batch * hq * nsplit > 0x7fffffffLL || (int64_t)hq * ntile > 0x7fffffffLL ||
      (int64_t)batch * hq * n_rows > 0x7fffffffLL)
    return SA_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  if (!isfinite(scale)) return SA_ERR_INVALID_ARG;
  *scale_out = scale;
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sa_sample_scores(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                           int32_t head_dim, int32_t dtype, float softmax_scale, int32_t row0, int32_t n_rows,
                           int32_t band, const uint8_t* skip_cols, int32_t lse_given, float* row_lse,
                           void* workspace, size_t workspace_bytes, int64_t* diag_score, int64_t* vert_score,
                           void* stream) {
  float scale = 0.0f;
  const sa_status st = sample_args_ok(q, k, batch, hq, hkv, S, head_dim, dtype, softmax_scale, row0, n_rows, band,
                                      row_lse, diag_score, vert_score, &scale);
  if (st != SA_OK) return st;
  if (!lse_given) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 7u)) return SA_ERR_INVALID_ARG;
    if (workspace_bytes < sa::sample_workspace_bytes(batch, hq, row0, n_rows)) return SA_ERR_CAPACITY;
  }
  return hip_status(sa::launch_sample_scores(q, k, batch, hq, hkv, S, head_dim, dtype, scale, row0, n_rows, band,
                                             skip_cols, lse_given != 0, row_lse, workspace, diag_score, vert_score,
                                             static_cast<hipStream_t>(stream)));
}

sa_status sa_sample_scores_noalloc(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t S,
                                   int32_t head_dim, int32_t dtype, float softmax_scale, int32_t row0, int32_t n_rows,
                                   int32_t band, const uint8_t* skip_cols, int32_t lse_given, float* row_lse,
                                   int64_t* diag_score, int64_t* vert_score, void* stream) {
  float scale = 0.0f;
  const sa_status st = sample_args_ok(q, k, batch, hq, hkv, S, head_dim, dtype, softmax_scale, row0, n_rows, band,
                                      row_lse, diag_score, vert_score, &scale);
  if (st != SA_OK) return st;
  void* ws = nullptr;
  if (!lse_given) {
    if (sa::sample_workspace_bytes(batch, hq, row0, n_rows) > sa::kSampleStaticScratchBytes) return SA_ERR_CAPACITY;
    if (sa::sample_static_scratch(&ws) != hipSuccess) return SA_ERR_HIP;
  }
  return hip_status(sa::launch_sample_scores(q, k, batch, hq, hkv, S, head_dim, dtype, scale, row0, n_rows, band,
                                             skip_cols, lse_given != 0, row_lse, ws, diag_score, vert_score,
                                             static_cast<hipStream_t>(stream)));
}

sa_status sa_select_patterns(const int64_t* scores, int32_t n_heads, int32_t S, double alpha, int64_t rows,
                             int32_t band, uint8_t* keep, void* stream) {
  if (!scores || !keep) return SA_ERR_INVALID_ARG;
  if (n_heads < 1 || S < 1 || band < 0) return SA_ERR_INVALID_ARG;
  if (!(alpha > 0.0 && alpha <= 1.0)) return SA_ERR_INVALID_ARG;
  if (rows < 1 || rows > ((int64_t)1 << 30)) return SA_ERR_INVALID_ARG;  // rows * 2^32 stays below 2^62
  if (reinterpret_cast<uintptr_t>(scores) & 7u) return SA_ERR_INVALID_ARG;
  return hip_status(sa::launch_select(scores, n_heads, S, alpha, rows << 32, band, keep,
                                      static_cast<hipStream_t>(stream)));
}

sa_status sa_calib_mfma_bf16(int32_t n_workgroups, int32_t iters, float* sink, void* stream) {
  if (!sink || n_workgroups < 1 || iters < 1) return SA_ERR_INVALID_ARG;
  return hip_status(sa::launch_calib_mfma(n_workgroups, iters, sink, static_cast<hipStream_t>(stream)));
}

sa_status sa_calib_gather(const void* buf, int64_t region_bytes, int32_t chunk_bytes, int32_t n_workgroups,
                          int32_t reads_per_workgroup, uint64_t seed, float* sink, void* stream) {
  if (!buf || !sink || n_workgroups < 1 || reads_per_workgroup < 1) return SA_ERR_INVALID_ARG;
  if (!aligned16(buf) || chunk_bytes < 16 || chunk_bytes % 16 != 0 || region_bytes < chunk_bytes)
    return SA_ERR_INVALID_ARG;
  return hip_status(sa::launch_calib_gather(buf, region_bytes, chunk_bytes, n_workgroups, reads_per_workgroup, seed,
                                            sink, static_cast<hipStream_t>(stream)));
}

sa_status sa_attention_maps(const void* q, const void* k, int32_t batch, int32_t hq, int32_t hkv, int32_t L,
                            int32_t head_dim, int32_t dtype, float softmax_scale, float* maps, void* stream) {
  if (!q || !k || !maps) return SA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(maps)) return SA_ERR_INVALID_ARG;
  if (batch < 1 || hq < 1 || hkv < 1 || L < 1 || hq % hkv != 0) return SA_ERR_INVALID_ARG;
  if (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F32) return SA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (L > sa::kMaxCaptureL) return SA_ERR_UNSUPPORTED;
  if ((int64_t)hq * ((L + 63) / 64) > 0x7fffffffLL) return SA_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  if (!isfinite(scale)) return SA_ERR_INVALID_ARG;
  return hip_status(sa::launch_attention_maps(q, k, batch, hq, hkv, L, head_dim, dtype, scale, maps,
                                              static_cast<hipStream_t>(stream)));
}

sa_status sa_patterns_to_desc(const uint8_t* keep_diag, const uint8_t* keep_vert, int32_t n_maps, int32_t L,
                              int32_t S, int32_t* diag_ptr, int32_t* diag_off, int32_t* vert_ptr, int32_t* vert_col,
                              void* stream) {
  if (!keep_diag || !keep_vert || !diag_ptr || !diag_off || !vert_ptr || !vert_col) return SA_ERR_INVALID_ARG;
  if (n_maps < 1 || L < 1 || S < 1) return SA_ERR_INVALID_ARG;
  return hip_status(sa::launch_patterns_to_desc(keep_diag, keep_vert, n_maps, L, S, diag_ptr, diag_off, vert_ptr,
                                                vert_col, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
