// C ABI of libdsa: argument validation, path selection and error reporting.
// Every check runs on the host before any launch; a rejected call writes nothing.
#include "dsa.h"

#include <atomic>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cmath>
#include <cstring>

#include "kernels.h"

static_assert(DSA_TOPK_NOALLOC_SCRATCH_BYTES == dsa::kTopkScratchBytes, "the header states the scratch size");

namespace {

thread_local char g_err[512] = "";
std::atomic<int> g_topk_path{0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int d) { return d == DSA_F32 || d == DSA_BF16 || d == DSA_F16; }

}  // namespace

extern "C" {

int dsa_version(void) { return 100; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size is out of range or inconsistent";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: unsupported dtype or dtype pairing";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: valid arguments outside the implemented set";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown libdsa status";
  }
}

const char* dsa_last_error(void) { return g_err; }

int dsa_layer_computes_topk(int layer) {
  if (layer < 0) return fail(DSA_ERR_SHAPE, "dsa_layer_computes_topk: layer=%d must be >= 0", layer);
  return (layer <= 1 || layer % 4 == 2) ? 1 : 0;
}

int dsa_topk_source_layer(int layer) {
  if (layer < 0) return fail(DSA_ERR_SHAPE, "dsa_topk_source_layer: layer=%d must be >= 0", layer);
  if (layer <= 1) return layer;
  return 4 * ((layer - 2) / 4) + 2;  // the most recent layer 4m + 2 at or below `layer`
}

int dsa_set_tuning(const char* key, int value) {
  if (!key) return fail(DSA_ERR_NULL, "dsa_set_tuning: key is NULL");
  if (std::strcmp(key, "topk_path") == 0) {
    if (value < 0 || value > 3) return fail(DSA_ERR_SHAPE, "topk_path must be 0..3 (got %d)", value);
    g_topk_path.store(value);
    return ok();
  }
  if (std::strcmp(key, "score_chunks_per_wave") == 0) {
    if (value < 0 || value > 64) return fail(DSA_ERR_SHAPE, "score_chunks_per_wave must be 0..64 (got %d)", value);
    dsa::g_score_cpw.store(value);
    return ok();
  }
  if (std::strcmp(key, "score_prefill_waves") == 0) {
    if (value != 0 && value != 4 && value != 8)
      return fail(DSA_ERR_SHAPE, "score_prefill_waves must be 0, 4 or 8 (got %d)", value);
    dsa::g_score_prefill_waves.store(value);
    return ok();
  }
  if (std::strcmp(key, "mla_tiles_per_step") == 0) {
    if (value < 0 || value > 3)
      return fail(DSA_ERR_SHAPE, "mla_tiles_per_step must be 0, 1, 2 or 3 (got %d)", value);
    dsa::g_mla_tiles_per_step.store(value);
    return ok();
  }
  if (std::strcmp(key, "topk_cand_block") == 0) {
    if (value != 0 && value != 256 && value != 512 && value != 1024)
      return fail(DSA_ERR_SHAPE, "topk_cand_block must be 0, 256, 512 or 1024 (got %d)", value);
    dsa::g_topk_cand_block.store(value);
    return ok();
  }
  if (std::strcmp(key, "mla_head_split") == 0) {
    if (value < 0 || value > 2) return fail(DSA_ERR_SHAPE, "mla_head_split must be 0, 1 or 2 (got %d)", value);
    dsa::g_mla_head_split.store(value);
    return ok();
  }
  return fail(DSA_ERR_SHAPE, "dsa_set_tuning: unknown key '%s'", key);
}

static int index_score_checked(const char* fn, const void* q, const void* k_cache, const float* w,
                               const int32_t* kv_len, const int32_t* q_pos, float* scores, int B, int n_q,
                               int H, int D, int n_kv, int q_dtype, int k_dtype, float scale,
                               dsa::ScoreArgs sink, hipStream_t stream, bool launch = true) {
  if (!q || !k_cache || !w || !scores)
    return fail(DSA_ERR_NULL, "%s: q, k_cache, w and scores must be non-NULL", fn);
  if (B < 1 || n_q < 1 || H < 1 || D < 1 || n_kv < 1)
    return fail(DSA_ERR_SHAPE, "%s: B=%d n_q=%d H=%d D=%d n_kv=%d must all be >= 1", fn, B, n_q, H, D, n_kv);
  if ((long long)B * n_q > INT_MAX || (long long)B * n_q * n_kv > (1LL << 40) || n_kv > (1 << 30))
    return fail(DSA_ERR_SHAPE, "%s: n_kv (at most 2^30) or B*n_q*n_kv too large", fn);
  if (!valid_dtype(q_dtype) || !valid_dtype(k_dtype))
    return fail(DSA_ERR_DTYPE, "%s: unknown dtype (q %d, k %d)", fn, q_dtype, k_dtype);
  if (q_dtype != k_dtype)
    return fail(DSA_ERR_DTYPE, "%s: q_dtype (%d) must equal k_dtype (%d)", fn, q_dtype, k_dtype);
  const bool mfma = D == 128 && H <= 32 && q_dtype != DSA_F32;
  // grid limits: the decode and plain kernels put B * n_q on the grid's y dimension, the
  // prefill kernel (16-bit, D = 128, n_q >= 8) puts B on its z dimension
  if ((mfma && n_q >= 8) ? B > 65535 : (long long)B * n_q > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "%s: B=%d n_q=%d exceed the launch grid (%s <= 65535)", fn, B, n_q,
                (mfma && n_q >= 8) ? "B" : "B * n_q");
  if (mfma && (!aligned16(q) || !aligned16(k_cache)))
    return fail(DSA_ERR_UNSUPPORTED, "%s: q and k_cache must be 16-byte aligned", fn);
  if (!mfma && (long long)H * D > 16384)
    return fail(DSA_ERR_UNSUPPORTED, "%s: H*D = %lld exceeds 16384 outside the MFMA shape (16-bit, D=128, H<=32)",
                fn, (long long)H * D);
  if (!launch) return DSA_OK;
  return hip_status(dsa::launch_index_score(q, k_cache, w, kv_len, q_pos, scores, B, n_q, H, D, n_kv, q_dtype,
                                            scale, sink, stream),
                    fn);
}

int dsa_index_score(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                    const int32_t* q_pos, float* scores, int B, int n_q, int H, int D, int n_kv,
                    int q_dtype, int k_dtype, float scale, hipStream_t stream) {
  return index_score_checked("dsa_index_score", q, k_cache, w, kv_len, q_pos, scores, B, n_q, H, D, n_kv,
                             q_dtype, k_dtype, scale, dsa::ScoreArgs{nullptr, 0, 0.f, 1}, stream);
}

int dsa_index_score_sink(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                         const int32_t* q_pos, const int32_t* sink_start, int n_sink, float sink_boost,
                         float* scores, int B, int n_q, int H, int D, int n_kv, int q_dtype, int k_dtype,
                         float scale, hipStream_t stream) {
  if (n_sink < 0) return fail(DSA_ERR_SHAPE, "dsa_index_score_sink: n_sink=%d must be >= 0", n_sink);
  if (!std::isfinite(sink_boost)) return fail(DSA_ERR_SHAPE, "dsa_index_score_sink: sink_boost must be finite");
  return index_score_checked("dsa_index_score_sink", q, k_cache, w, kv_len, q_pos, scores, B, n_q, H, D, n_kv,
                             q_dtype, k_dtype, scale, dsa::ScoreArgs{sink_start, n_sink, sink_boost, 1}, stream);
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the fused call: the candidates (fused path) or the top-k workspace (score and
// top-k one after the other), then the score rows when the caller passes no score array.
static size_t score_topk_bytes(const dsa::ScoreTopkPlan& p, int B, int n_q, int n_kv, int top_k,
                               bool scores_in_ws) {
  const long rows = (long)B * n_q;
  const size_t sel = p.ok ? p.cand_bytes : dsa::plan_topk((int)rows, n_kv, top_k, 0).ws_bytes;
  return align256(sel) + (scores_in_ws ? align256((size_t)rows * n_kv * sizeof(float)) : 0);
}

size_t dsa_index_score_topk_workspace_size(int B, int n_q, int H, int D, int n_kv, int top_k, int dtype,
                                           int scores_in_workspace) {
  if (B < 1 || n_q < 1 || H < 1 || D < 1 || n_kv < 1 || top_k < 1 || (long long)B * n_q > 65535) return 0;
  return score_topk_bytes(dsa::plan_score_topk(B, n_q, H, D, n_kv, top_k, dtype), B, n_q, n_kv, top_k,
                          scores_in_workspace != 0);
}

int dsa_index_score_topk(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                         const int32_t* q_pos, float* scores, int32_t* idx, int B, int n_q, int H, int D, int n_kv,
                         int top_k, int q_dtype, int k_dtype, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const char* fn = "dsa_index_score_topk";
  if (!q || !k_cache || !w || !idx) return fail(DSA_ERR_NULL, "%s: q, k_cache, w and idx must be non-NULL", fn);
  if (top_k < 1) return fail(DSA_ERR_SHAPE, "%s: top_k=%d must be >= 1", fn, top_k);
  if (B >= 1 && n_q >= 1 && (long long)B * n_q > 65535)
    return fail(DSA_ERR_SHAPE, "%s: B * n_q = %lld rows exceed 65535", fn, (long long)B * n_q);
  // the score arguments are checked as dsa_index_score checks them, without launching (a NULL
  // score array is allowed here: the workspace then holds the scores)
  if (const int st = index_score_checked(fn, q, k_cache, w, kv_len, q_pos, scores ? scores : const_cast<float*>(w), B,
                                         n_q, H, D, n_kv, q_dtype, k_dtype, scale,
                                         dsa::ScoreArgs{nullptr, 0, 0.f, 1}, stream, false))
    return st;
  const dsa::ScoreTopkPlan plan = dsa::plan_score_topk(B, n_q, H, D, n_kv, top_k, q_dtype);
  const size_t need = score_topk_bytes(plan, B, n_q, n_kv, top_k, scores == nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                workspace ? "" : " (NULL)");
  const int rows = B * n_q;
  char* ws = static_cast<char*>(workspace);
  const size_t sel_bytes = align256(plan.ok ? plan.cand_bytes : dsa::plan_topk(rows, n_kv, top_k, 0).ws_bytes);
  float* sc = scores ? scores : reinterpret_cast<float*>(ws + sel_bytes);
  if (!plan.ok) {  // score, then top-k over the stored rows
    hipError_t e = dsa::launch_index_score(q, k_cache, w, kv_len, q_pos, sc, B, n_q, H, D, n_kv, q_dtype, scale,
                                           dsa::ScoreArgs{nullptr, 0, 0.f, 1}, stream);
    if (e != hipSuccess) return hip_status(e, "dsa_index_score_topk score launch");
    const dsa::TopkPlan tp = dsa::plan_topk(rows, n_kv, top_k, g_topk_path.load());
    return hip_status(dsa::launch_topk(sc, idx, rows, n_kv, top_k, tp, ws, stream), "dsa_index_score_topk top-k launch");
  }
  const size_t slots = (size_t)rows * plan.n_w * plan.m;
  dsa::CandOut cand{reinterpret_cast<uint2*>(ws), reinterpret_cast<uint4*>(ws + align256(slots * 8)), plan.m};
  hipError_t e = dsa::launch_index_score_cand(q, k_cache, w, kv_len, q_pos, sc, B, n_q, H, n_kv, q_dtype, scale, plan,
                                              cand, stream);
  if (e != hipSuccess) return hip_status(e, "dsa_index_score_topk score launch");
  return hip_status(dsa::launch_topk_cand(sc, idx, rows, n_kv, top_k, plan, cand, stream),
                    "dsa_index_score_topk select launch");
}

size_t dsa_topk_workspace_size(int rows, int n_kv, int top_k) {
  if (rows < 1 || n_kv < 1 || top_k < 1) return 0;
  return dsa::plan_topk(rows, n_kv, top_k, 0).ws_bytes;
}

static int topk_args(const char* fn, const float* scores, const int32_t* idx, int rows, int n_kv, int top_k) {
  if (!scores || !idx) return fail(DSA_ERR_NULL, "%s: scores and idx must be non-NULL", fn);
  if (rows < 1 || n_kv < 1 || top_k < 1)
    return fail(DSA_ERR_SHAPE, "%s: rows=%d n_kv=%d top_k=%d must all be >= 1", fn, rows, n_kv, top_k);
  if ((long long)rows * n_kv > (1LL << 40) || rows > 65535)
    return fail(DSA_ERR_SHAPE, "%s: rows=%d x n_kv=%d out of range (rows <= 65535)", fn, rows, n_kv);
  return DSA_OK;
}

int dsa_topk(const float* scores, int32_t* idx, int rows, int n_kv, int top_k, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  if (const int st = topk_args("dsa_topk", scores, idx, rows, n_kv, top_k)) return st;
  const size_t need = dsa_topk_workspace_size(rows, n_kv, top_k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_topk: workspace of %zu bytes needed, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  const dsa::TopkPlan plan = dsa::plan_topk(rows, n_kv, top_k, g_topk_path.load());
  return hip_status(dsa::launch_topk(scores, idx, rows, n_kv, top_k, plan, workspace, stream),
                    "dsa_topk launch");
}

int dsa_topk_noalloc(const float* scores, int32_t* idx, int rows, int n_kv, int top_k, hipStream_t stream) {
  if (const int st = topk_args("dsa_topk_noalloc", scores, idx, rows, n_kv, top_k)) return st;
  const size_t need = dsa_topk_workspace_size(rows, n_kv, top_k);
  if (need > dsa::kTopkScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_topk_noalloc: this shape needs %zu bytes of scratch and the library's static array holds "
                "%zu; call dsa_topk with a workspace",
                need, dsa::kTopkScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = dsa::topk_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "dsa_topk_noalloc: scratch address");
  }
  const dsa::TopkPlan plan = dsa::plan_topk(rows, n_kv, top_k, g_topk_path.load());
  return hip_status(dsa::launch_topk(scores, idx, rows, n_kv, top_k, plan, ws, stream), "dsa_topk_noalloc launch");
}

int dsa_sparse_mla_num_splits(int B, int n_q, int top_k) {
  if (B < 1 || n_q < 1 || top_k < 1) return 1;
  return dsa::mla_auto_splits(B, n_q, top_k);
}

size_t dsa_sparse_mla_workspace_size(int B, int n_q, int Hm, int top_k, int d_latent, int n_split) {
  if (B < 1 || n_q < 1 || Hm < 1 || top_k < 1 || d_latent < 1) return 0;
  if (n_split <= 0) n_split = dsa::mla_auto_splits(B, n_q, top_k);
  if (n_split > top_k) n_split = top_k;
  return dsa::mla_workspace_bytes(B, n_q, Hm, top_k, d_latent, n_split);
}

int dsa_sparse_mla_attn(const void* q_abs, const void* latent, const int32_t* idx,
                        const int32_t* kv_len, float* out, float* lse, int B, int n_q, int Hm,
                        int n_kv, int top_k, int d_latent, int d_rope, float sm_scale, int dtype,
                        int n_split, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q_abs || !latent || !idx || !out)
    return fail(DSA_ERR_NULL, "dsa_sparse_mla_attn: q_abs, latent, idx and out must be non-NULL");
  if (B < 1 || n_q < 1 || Hm < 1 || n_kv < 1 || top_k < 1 || d_latent < 1 || d_rope < 0)
    return fail(DSA_ERR_SHAPE,
                "dsa_sparse_mla_attn: B=%d n_q=%d Hm=%d n_kv=%d top_k=%d d_latent=%d d_rope=%d out of range",
                B, n_q, Hm, n_kv, top_k, d_latent, d_rope);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_DTYPE, "dsa_sparse_mla_attn: dtype must be F32 or BF16 (got %d)", dtype);
  if (n_split <= 0) n_split = dsa::mla_auto_splits(B, n_q, top_k);
  if (n_split > top_k) n_split = top_k;
  if ((long long)B * n_q * n_split * Hm > INT_MAX)
    return fail(DSA_ERR_SHAPE, "dsa_sparse_mla_attn: B*n_q*n_split*Hm too large");
  const int chunk = (top_k + n_split - 1) / n_split;
  const bool mfma = dsa::mla_mfma_supported(Hm, d_latent, d_rope, dtype);
  if (mfma) {
    if (chunk > 2048)
      return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_attn: %d index slots per part exceed 2048; use n_split >= %d",
                  chunk, (top_k + 2047) / 2048);
    if (!aligned16(q_abs) || !aligned16(latent) || !aligned16(out))
      return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_attn: q_abs, latent and out must be 16-byte aligned");
  } else if ((long long)B * n_q > 65535) {
    return fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_attn: B * n_q = %lld exceeds the plain kernel's launch grid "
                "(<= 65535 outside the MFMA shape)", (long long)B * n_q);
  } else if (d_latent + d_rope > 1024 || d_latent > 1024) {
    return fail(DSA_ERR_UNSUPPORTED,
                "dsa_sparse_mla_attn: d_latent + d_rope = %d exceeds 1024 outside the MFMA shape "
                "(bf16, Hm %% 16 == 0, Hm <= 64, d_latent 512, d_rope 0 or 64)",
                d_latent + d_rope);
  }
  const size_t need = dsa::mla_workspace_bytes(B, n_q, Hm, top_k, d_latent, n_split);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_mla_attn: workspace of %zu bytes needed, got %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  return hip_status(dsa::launch_sparse_mla(q_abs, latent, idx, kv_len, out, lse, B, n_q, Hm, n_kv, top_k,
                                           d_latent, d_rope, sm_scale, dtype, n_split, workspace, stream),
                    "dsa_sparse_mla_attn launch");
}

int dsa_indexer_prep(const float* q_in, const float* k_in, const void* latent_in, const int32_t* pos,
                     void* q_out, void* k_cache, void* latent_cache, int B, int n_new, int H, int n_kv,
                     int row_bytes, int out_dtype, float rope_base, int hadamard, hipStream_t stream) {
  if (!pos) return fail(DSA_ERR_NULL, "dsa_indexer_prep: pos must be non-NULL");
  if (!q_in && !k_in && !latent_in)
    return fail(DSA_ERR_NULL, "dsa_indexer_prep: one of q_in, k_in, latent_in must be non-NULL");
  if (!q_in != !q_out || !k_in != !k_cache || !latent_in != !latent_cache)
    return fail(DSA_ERR_NULL, "dsa_indexer_prep: q_in/q_out, k_in/k_cache and latent_in/latent_cache "
                              "must be given in pairs");
  if (B < 1 || n_new < 1 || n_kv < 1 || (q_in && (H < 1 || H > 65536)))
    return fail(DSA_ERR_SHAPE, "dsa_indexer_prep: B=%d n_new=%d H=%d n_kv=%d out of range", B, n_new, H, n_kv);
  if ((long long)B * n_new * (q_in ? H + 1 : 1) > INT_MAX || (long long)B * n_kv > (1LL << 34))
    return fail(DSA_ERR_SHAPE, "dsa_indexer_prep: too many rows");
  if (latent_in && (row_bytes < 16 || row_bytes % 16 != 0))
    return fail(DSA_ERR_SHAPE, "dsa_indexer_prep: row_bytes=%d must be a positive multiple of 16", row_bytes);
  if (!valid_dtype(out_dtype)) return fail(DSA_ERR_DTYPE, "dsa_indexer_prep: unknown out_dtype %d", out_dtype);
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(DSA_ERR_SHAPE, "dsa_indexer_prep: rope_base must be positive and finite");
  const void* ptrs[] = {q_in, k_in, latent_in, q_out, k_cache, latent_cache};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DSA_ERR_UNSUPPORTED, "dsa_indexer_prep: pointers must be 16-byte aligned");
  return hip_status(dsa::launch_indexer_prep(q_in, k_in, latent_in, pos, q_out, k_cache, latent_cache, B, n_new,
                                             q_in ? H : 1, n_kv, row_bytes, out_dtype, std::log2((double)rope_base),
                                             hadamard != 0, stream),
                    "dsa_indexer_prep launch");
}

int dsa_kpool_compress(const void* packed, int row_stride, int row_dtype, const float* ape, void* pooled,
                       int out_dtype, int B, int n_kv, int D, int kpool, int pool_begin, int pool_end,
                       hipStream_t stream) {
  if (!packed || !ape || !pooled)
    return fail(DSA_ERR_NULL, "dsa_kpool_compress: packed, ape and pooled must be non-NULL");
  if (B < 1 || n_kv < 1 || D < 1 || D > 4096 || kpool < 1 || kpool > 8 || row_stride < 2 * D + 1)
    return fail(DSA_ERR_SHAPE, "dsa_kpool_compress: B=%d n_kv=%d D=%d kpool=%d row_stride=%d out of range "
                               "(D <= 4096, 1 <= kpool <= 8, row_stride >= 2 D + 1)", B, n_kv, D, kpool, row_stride);
  if (B > 65535 || (long long)B * n_kv * row_stride > (1LL << 40))
    return fail(DSA_ERR_SHAPE, "dsa_kpool_compress: cache too large");
  if (pool_begin < 0 || pool_end < pool_begin || pool_end > n_kv / kpool)
    return fail(DSA_ERR_SHAPE, "dsa_kpool_compress: pools [%d, %d) outside [0, %d)", pool_begin, pool_end,
                n_kv / kpool);
  if ((long long)(pool_end - pool_begin) * D > INT_MAX)
    return fail(DSA_ERR_SHAPE, "dsa_kpool_compress: (pool_end - pool_begin) * D above 2^31 - 1 per call");
  if (!valid_dtype(row_dtype) || !valid_dtype(out_dtype))
    return fail(DSA_ERR_DTYPE, "dsa_kpool_compress: unknown dtype (rows %d, pooled %d)", row_dtype, out_dtype);
  return hip_status(dsa::launch_kpool_compress(packed, row_stride, row_dtype, ape, pooled, out_dtype, B, n_kv, D,
                                               kpool, pool_begin, pool_end, stream),
                    "dsa_kpool_compress launch");
}

int dsa_kpool_index_score(const void* q, const void* pooled, const float* w, const int32_t* kv_len,
                          const int32_t* q_pos, float* scores, int B, int n_q, int H, int D, int n_pool,
                          int kpool, int q_dtype, int k_dtype, float scale, hipStream_t stream) {
  if (kpool < 1 || kpool > 8)
    return fail(DSA_ERR_SHAPE, "dsa_kpool_index_score: kpool=%d must be in [1, 8]", kpool);
  return index_score_checked("dsa_kpool_index_score", q, pooled, w, kv_len, q_pos, scores, B, n_q, H, D, n_pool,
                             q_dtype, k_dtype, scale, dsa::ScoreArgs{nullptr, 0, 0.f, kpool}, stream);
}

int dsa_kpool_expand(const int32_t* pool_idx, const void* packed, int row_stride, int row_dtype, int D,
                     const int32_t* kv_len, const int32_t* q_pos, int32_t* tok_idx, int B, int n_q, int n_kv,
                     int top_pools, int kpool, hipStream_t stream) {
  if (!pool_idx || !packed || !tok_idx)
    return fail(DSA_ERR_NULL, "dsa_kpool_expand: pool_idx, packed and tok_idx must be non-NULL");
  if (B < 1 || n_q < 1 || n_kv < 1 || D < 1 || top_pools < 1 || kpool < 1 || kpool > 8 || row_stride < 2 * D + 1)
    return fail(DSA_ERR_SHAPE, "dsa_kpool_expand: B=%d n_q=%d n_kv=%d D=%d top_pools=%d kpool=%d row_stride=%d "
                               "out of range", B, n_q, n_kv, D, top_pools, kpool, row_stride);
  if ((long long)B * n_q > 65535 || (long long)kpool * top_pools + kpool - 1 > (1 << 24) ||
      (long long)B * n_kv * row_stride > (1LL << 40))
    return fail(DSA_ERR_SHAPE, "dsa_kpool_expand: B * n_q (<= 65535), width or cache too large");
  if (!valid_dtype(row_dtype)) return fail(DSA_ERR_DTYPE, "dsa_kpool_expand: unknown row dtype %d", row_dtype);
  return hip_status(dsa::launch_kpool_expand(pool_idx, packed, row_stride, row_dtype, D, kv_len, q_pos, tok_idx,
                                             B, n_q, n_kv, top_pools, kpool, stream),
                    "dsa_kpool_expand launch");
}

int dsa_kpool_sparse_mla_attn(const void* q_abs, const void* latent, const int32_t* pool_idx, const void* packed,
                              int row_stride, int row_dtype, int D, const int32_t* kv_len, const int32_t* q_pos,
                              float* out, float* lse, int B, int n_q, int Hm, int n_kv, int top_pools, int kpool,
                              int d_latent, int d_rope, float sm_scale, int dtype, int n_split, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_kpool_sparse_mla_attn";
  if (!q_abs || !latent || !pool_idx || !packed || !out)
    return fail(DSA_ERR_NULL, "%s: q_abs, latent, pool_idx, packed and out must be non-NULL", fn);
  if (B < 1 || n_q < 1 || Hm < 1 || n_kv < 1 || D < 1 || top_pools < 1 || kpool < 1 || kpool > 8 ||
      row_stride < 2 * D + 1 || d_latent < 1 || d_rope < 0)
    return fail(DSA_ERR_SHAPE, "%s: B=%d n_q=%d Hm=%d n_kv=%d D=%d top_pools=%d kpool=%d row_stride=%d "
                               "d_latent=%d d_rope=%d out of range", fn, B, n_q, Hm, n_kv, D, top_pools, kpool,
                row_stride, d_latent, d_rope);
  const long long width = (long long)kpool * top_pools + kpool - 1;
  if (width > (1 << 24) || (long long)B * n_kv * row_stride > (1LL << 40))
    return fail(DSA_ERR_SHAPE, "%s: kpool * top_pools or the packed cache too large", fn);
  if (!valid_dtype(row_dtype)) return fail(DSA_ERR_DTYPE, "%s: unknown row dtype %d", fn, row_dtype);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_DTYPE, "%s: dtype must be F32 or BF16 (got %d)", fn, dtype);
  if (!dsa::mla_mfma_supported(Hm, d_latent, d_rope, dtype))
    return fail(DSA_ERR_UNSUPPORTED, "%s: only the MFMA attention shapes (bf16, Hm %% 16 == 0, Hm <= 64, "
                                     "d_latent 512, d_rope 0 or 64); use dsa_kpool_expand + dsa_sparse_mla_attn", fn);
  const int top_k = (int)width;
  if (n_split <= 0) n_split = dsa::mla_auto_splits(B, n_q, top_k);
  if (n_split > top_k) n_split = top_k;
  if ((long long)B * n_q * n_split * Hm > INT_MAX) return fail(DSA_ERR_SHAPE, "%s: B*n_q*n_split*Hm too large", fn);
  const int chunk = (top_k + n_split - 1) / n_split;
  if (chunk > 2048)
    return fail(DSA_ERR_UNSUPPORTED, "%s: %d index slots per part exceed 2048; use n_split >= %d", fn, chunk,
                (top_k + 2047) / 2048);
  if (!aligned16(q_abs) || !aligned16(latent) || !aligned16(out))
    return fail(DSA_ERR_UNSUPPORTED, "%s: q_abs, latent and out must be 16-byte aligned", fn);
  const int esz = row_dtype == DSA_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(packed) & (uintptr_t)(esz - 1)) != 0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: packed must be aligned to its element size", fn);
  const size_t need = dsa::mla_workspace_bytes(B, n_q, Hm, top_k, d_latent, n_split);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                workspace ? "" : " (NULL)");
  const dsa::KpoolSlots ks{pool_idx, static_cast<const uint8_t*>(packed), (long)row_stride * esz, 2 * D * esz,
                           row_dtype == DSA_F32 ? 1 : 0, top_pools, kpool, q_pos};
  return hip_status(dsa::launch_sparse_mla(q_abs, latent, nullptr, kv_len, out, lse, B, n_q, Hm, n_kv, top_k,
                                           d_latent, d_rope, sm_scale, dtype, n_split, workspace, stream, &ks),
                    "dsa_kpool_sparse_mla_attn launch");
}

}  // extern "C"

