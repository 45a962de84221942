/*
 * libdsa — DeepSeek Sparse Attention (DSA) hot path for AMD Instinct MI355X (gfx950).
 *
 * Three calls, one per step of the method, run back to back on one HIP stream:
 *
 *   dsa_index_score      lightning-indexer scores of each query against every cached key
 *   dsa_topk             the top_k highest-scoring cache rows of each query
 *   dsa_sparse_mla_attn  absorbed MLA attention over only the selected 576-wide latent rows
 *
 * Conventions shared by every call:
 *   - Pointers named as device buffers must be device memory (hipMalloc, or a torch
 *     tensor on the GPU). The caller owns every buffer; the library never allocates,
 *     frees or keeps a pointer beyond the call. Scratch memory is a caller-provided
 *     workspace whose size the matching *_workspace_size query returns.
 *   - Arrays are dense and row-major with the shapes written next to each argument.
 *   - Every call returns a status (DSA_OK or a negative DSA_ERR_*). Argument errors are
 *     detected on the host before anything is launched; the call then writes nothing.
 *     DSA_ERR_HIP reports a failed kernel launch. No call synchronises the host or the
 *     stream: faults inside a kernel surface at the caller's next synchronisation.
 *   - Calls keep no state from one call to the next and may be made from several host
 *     threads at once (dsa_last_error is per thread). The one process-wide state is the
 *     set of tuning switches of dsa_set_tuning: each call reads them once when it starts,
 *     they only choose between kernels that give the results stated for the call, and
 *     they may be changed from any thread. Two calls that share a workspace must not
 *     overlap in time on the device.
 *   - bf16 and f16 data are 16-bit IEEE bit patterns (bfloat16: top half of an fp32).
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_F16 = 2 } dsa_dtype;

enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
  DSA_ERR_DTYPE = -3,       /* unknown dtype, or a dtype pairing the call does not take */
  DSA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than *_workspace_size */
  DSA_ERR_UNSUPPORTED = -5, /* valid arguments outside what the kernels implement */
  DSA_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed */
};

/*
 * Lightning-indexer score (ik_llama_opt commit log, sub-commit "Add GLM-5.2/DeepSeek-V3.2
 * DSA lightning indexer": relu(k.q) per indexer head, scaled by per-head weights, summed
 * over heads, plus the causal mask; sub-commit "decode-correct via persistent indexer-K
 * cache": every query is scored against all cached indexer keys).
 *
 *   scores[b][i][t] = scale * sum_h w[b][i][h] * max(0, sum_d q[b][i][h][d] * k_cache[b][t][d])
 *   scores[b][i][t] = -inf  where t > q_pos[b][i] or t >= kv_len[b]
 *
 * q        device, [B][n_q][H][D], q_dtype
 * k_cache  device, [B][n_kv][D], k_dtype (keys already roped and Hadamard-rotated upstream)
 * w        device, [B][n_q][H] fp32 per-head weights
 * kv_len   device, [B] int32 valid rows per sequence, or NULL (every sequence has n_kv)
 * q_pos    device, [B][n_q] int32 cache position of each query, or NULL
 *          (NULL: q_pos[b][i] = kv_len[b] - n_q + i, the queries are the last n_q rows)
 * scores   device, [B][n_q][n_kv] fp32, written in full
 * scale    factor applied after the head sum
 * Sizes: B, n_q, H, D, n_kv >= 1, n_kv <= 2^30. q_dtype must equal k_dtype (F32, BF16 or F16).
 * bf16/f16 with D = 128 and H <= 32 run on MFMA; other shapes run a plain kernel that
 * needs H * D <= 16384. Launch grid: B * n_q <= 65535, except on MFMA with n_q >= 8 (the
 * prefill kernel), where B <= 65535; larger shapes return DSA_ERR_UNSUPPORTED.
 */
int dsa_index_score(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                    const int32_t* q_pos, float* scores, int B, int n_q, int H, int D, int n_kv,
                    int q_dtype, int k_dtype, float scale, hipStream_t stream);

/*
 * dsa_index_score with the attention-sink boost (ik_llama_opt log: "DSA_SINK" force-inclusion
 * in the persistent-cache sub-commit, "per-sequence attention sink" and "UPDATE 6"
 * sub-commits: the first n_sink keys of the query's own sequence, counted from the sequence's
 * first present position, get a large additive boost so that top-k always keeps them):
 *
 *   scores[b][i][t] += sink_boost  for sink_start[b] <= t < sink_start[b] + n_sink, t not masked
 *
 * (the addition is a float32 add to the finished score; masked keys stay -inf). sink_start:
 * device [B] int32, each sequence's first present position, or NULL for 0 in every sequence.
 * n_sink >= 0 (0: same as dsa_index_score); sink_boost finite (the pages use 1e20, far above
 * any score, so the boosted keys tie and top-k keeps the lower positions first). Every other
 * argument and rule is that of dsa_index_score.
 */
int dsa_index_score_sink(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                         const int32_t* q_pos, const int32_t* sink_start, int n_sink, float sink_boost,
                         float* scores, int B, int n_q, int H, int D, int n_kv, int q_dtype, int k_dtype,
                         float scale, hipStream_t stream);

/*
 * Top-k selection (ik_llama_opt "DSA lightning indexer" sub-commit: top_k of
 * min(top_k, n_tokens), used as a set; "persistent indexer-K cache" sub-commit: the same
 * set from a descending argsort).
 *
 * For each row, the K = min(top_k, n_valid) largest valid scores, where NaN and -inf are
 * not valid and +inf is. Order: score descending, ties to the lower index; -0.0 equals
 * +0.0. idx[r] holds the chosen indices in ascending order followed by -1 up to top_k.
 * The result is unique, so it does not depend on the path or on timing.
 *
 * scores     device, [rows][n_kv] fp32
 * idx        device, [rows][top_k] int32, written in full
 * workspace  device scratch of at least dsa_topk_workspace_size(rows, n_kv, top_k) bytes
 *            (NULL allowed when that size is 0)
 * Sizes: rows >= 1, n_kv >= 1, top_k >= 1 (top_k > n_kv is allowed).
 */
size_t dsa_topk_workspace_size(int rows, int n_kv, int top_k);
int dsa_topk(const float* scores, int32_t* idx, int rows, int n_kv, int top_k, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/*
 * Fused score -> top-k (ik_llama_opt log, "decode-correct via persistent indexer-K cache":
 * every cached key is scored, then the top_k are taken; the two steps of dsa_index_score and
 * dsa_topk in one call). Results are exactly those of dsa_index_score followed by dsa_topk
 * over its scores: the same scores (bit for bit) and the same idx.
 *
 * For decode rows (bf16/f16, D = 128, H <= 32, n_q < 8) the scoring kernel also writes, for
 * each wave's range of keys, that range's largest keys as candidates, and one selection kernel
 * takes the top-k from their union; it reads a range's stored scores again only where the
 * range held more of the answer than it kept, and the whole row only when that set outgrows
 * one workgroup. So the score rows are written but, in the common case, not read back, and the
 * separate filter pass of dsa_topk is gone. Other shapes run dsa_index_score then dsa_topk.
 *
 * Arguments as in dsa_index_score, plus:
 * scores     device, [B][n_q][n_kv] fp32 out, or NULL (the workspace then holds the scores)
 * idx        device, [B][n_q][top_k] int32 out, as dsa_topk writes it
 * top_k      >= 1 (top_k > n_kv allowed)
 * workspace  device scratch of at least dsa_index_score_topk_workspace_size(B, n_q, H, D, n_kv,
 *            top_k, q_dtype, scores == NULL) bytes
 * B * n_q <= 65535.
 */
size_t dsa_index_score_topk_workspace_size(int B, int n_q, int H, int D, int n_kv, int top_k, int dtype,
                                           int scores_in_workspace);
int dsa_index_score_topk(const void* q, const void* k_cache, const float* w, const int32_t* kv_len,
                         const int32_t* q_pos, float* scores, int32_t* idx, int B, int n_q, int H, int D, int n_kv,
                         int top_k, int q_dtype, int k_dtype, float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * dsa_topk for callers that cannot allocate: code under HIP graph capture, tight serving
 * loops, and harnesses that forbid hipMalloc. It computes exactly what dsa_topk computes (the
 * same kernels, so the same idx), but takes no workspace: it uses a static device array of
 * DSA_TOPK_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it runs on until
 * the process ends, and calls no allocating routine. The array keeps the last call's contents;
 * nothing in it needs clearing between calls. All calls on one GPU share its array, so two
 * calls that overlap in time on one GPU (other streams, other host threads) race: order them.
 * Returns DSA_ERR_UNSUPPORTED, writing nothing, when dsa_topk_workspace_size(rows, n_kv, top_k)
 * exceeds the array (call dsa_topk with a workspace then); other arguments and errors as in
 * dsa_topk. The first call on a device looks up the array's address there (DSA_ERR_HIP if that
 * fails).
 */
#define DSA_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int dsa_topk_noalloc(const float* scores, int32_t* idx, int rows, int n_kv, int top_k, hipStream_t stream);

/*
 * Sparse absorbed MLA over the selected latent rows (ds4 "hy3: Metal decode path" PR,
 * GLM CPU oracle section: cached rows are 512 latent + 64 already-rotated rope values,
 * one softmax over the candidate rows; ik_llama_opt "MLA tensor parallelism" sub-commit:
 * absorbed per-head wk_b / wv_b; ds4 "Hy3 (295B)" PR: single-pass online softmax).
 *
 *   z[j]    = sm_scale * sum_{d < Dc} q_abs[b][i][h][d] * latent[b][j][d],  Dc = d_latent + d_rope
 *   out[b][i][h][:] = sum_j softmax(z)[j] * latent[b][j][0:d_latent]
 *   lse[b][i][h]    = log sum_j exp(z[j])
 * over the rows j = idx[b][i][s] with 0 <= j < kv_len[b] (other entries, e.g. -1, skip).
 * An empty selection gives out = 0 and lse = -inf.
 *
 * The selected rows are processed in n_split parts of ceil(top_k / n_split) index slots
 * each (online softmax inside a part) and the parts are merged by log-sum-exp.
 *
 * q_abs      device, [B][n_q][Hm][Dc], dtype
 * latent     device, [B][n_kv][Dc], dtype
 * idx        device, [B][n_q][top_k] int32
 * kv_len     device, [B] int32, or NULL (every sequence has n_kv valid rows)
 * out        device, [B][n_q][Hm][d_latent] fp32, written in full
 * lse        device, [B][n_q][Hm] fp32, or NULL
 * n_split    number of parts; <= 0 picks dsa_sparse_mla_num_splits(B, n_q, top_k)
 * workspace  device scratch of at least dsa_sparse_mla_workspace_size(...) bytes with the
 *            same B, n_q, Hm, top_k, d_latent, n_split (NULL allowed when that is 0)
 * dtype: F32 or BF16. BF16 with Hm a multiple of 16 (<= 64), d_latent = 512 and
 * d_rope in {0, 64} runs on MFMA; other shapes run a plain kernel that needs
 * Dc <= 1024, d_latent <= 1024 and B * n_q <= 65535 (DSA_ERR_UNSUPPORTED otherwise).
 *
 * dsa_sparse_mla_num_splits: the automatic part count, a host-side rule (no device work):
 * floor(256 / (B n_q)) parts, or floor(192 / (B n_q)) when parts would hold fewer than 400
 * slots, at most top_k / 128 (short selections: up to 4 parts of 16 slots or more) and at
 * least ceil(top_k / 2048); never fewer than 1.
 */
int dsa_sparse_mla_num_splits(int B, int n_q, int top_k);
size_t dsa_sparse_mla_workspace_size(int B, int n_q, int Hm, int top_k, int d_latent, int n_split);
int dsa_sparse_mla_attn(const void* q_abs, const void* latent, const int32_t* idx,
                        const int32_t* kv_len, float* out, float* lse, int B, int n_q, int Hm,
                        int n_kv, int top_k, int d_latent, int d_rope, float sm_scale, int dtype,
                        int n_split, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Indexer inputs of newly appended tokens (ik_llama_opt "DSA lightning indexer" sub-commit:
 * the indexer q and k split into a 64-dim rope part and a 64-dim nope part, NeoX rope on the
 * rope part, concatenated again; "persistent indexer-K cache" sub-commit: q and k are
 * Hadamard-rotated and the batch's keys are written into the key cache at their positions).
 * For each new token n at position p = pos[b][n]:
 *
 *   rope:      y[i]    = x[i] cos(a_i) - x[i+32] sin(a_i),   y[i+32] = x[i+32] cos(a_i) + x[i] sin(a_i),
 *              a_i = p * rope_base^(-i/32) for i < 32; dims 64..127 pass through
 *   rotation:  z = H y / sqrt(128), H the 128 x 128 Sylvester Hadamard matrix (if hadamard != 0)
 *   outputs:   q_out[b][n][h][:] = z(q_in[b][n][h][:]);  k_cache[b][p][:] = z(k_in[b][n][:]);
 *              latent_cache[b][p][:] = latent_in[b][n][:] (copied unchanged)
 *
 * q_in          device, [B][n_new][H][128] fp32, or NULL (no query output)
 * q_out         device, [B][n_new][H][128] out_dtype; NULL exactly when q_in is NULL
 * k_in          device, [B][n_new][128] fp32, or NULL (no key appended)
 * k_cache       device, [B][n_kv][128] out_dtype; rows pos[b][n] are written, no others;
 *               NULL exactly when k_in is NULL
 * latent_in     device, [B][n_new][row_bytes] raw rows (the 576-wide latent rows, any dtype),
 *               or NULL (no latent row appended)
 * latent_cache  device, [B][n_kv][row_bytes]; rows pos[b][n] are written; NULL exactly when
 *               latent_in is NULL
 * pos           device, [B][n_new] int32. A position outside [0, n_kv) writes no cache row
 *               (the query is still roped with it). Two new tokens of one sequence with the
 *               same position race.
 * out_dtype     F32, BF16 or F16 (rounded to nearest even from fp32)
 * row_bytes     bytes per latent row, a multiple of 16 (1152 for 576 bf16); ignored when
 *               latent_in is NULL
 * rope_base     the rope frequency base (> 0, finite)
 * Sizes: B, n_new, n_kv >= 1; 1 <= H <= 65536 when q_in is given; head dim 128 with 64 rope dims.
 * Pointers to 16-byte aligned memory. At least one of q_in, k_in, latent_in is non-NULL.
 */
int dsa_indexer_prep(const float* q_in, const float* k_in, const void* latent_in, const int32_t* pos,
                     void* q_out, void* k_cache, void* latent_cache, int B, int n_new, int H, int n_kv,
                     int row_bytes, int out_dtype, float rope_base, int hadamard, hipStream_t stream);

/*
 * IndexShare layer map (ik_llama_opt log, "GLM-5.2 DSA: IndexShare" sub-commit): in a model
 * with n_layer DSA layers, "full" layers compute their own scores and top-k, and every
 * "shared" layer reuses the indices of the most recent full layer (pass the same idx array to
 * dsa_sparse_mla_attn). A layer is full iff layer <= 1 or layer % 4 == 2 (21 of GLM-5.2's 78).
 * Returns 1 for a full layer, 0 for a shared one, DSA_ERR_SHAPE for layer < 0.
 */
int dsa_layer_computes_topk(int layer);
/* The full layer whose indices layer `layer` uses (itself when full), or DSA_ERR_SHAPE. */
int dsa_topk_source_layer(int layer);

/*
 * Tuning switches. They choose between kernels that compute identical results and
 * change only speed. key "topk_path": 0 = automatic, 1 = one workgroup per row,
 * 2 = two-stage (segments, then candidates), 3 = filtered (a sampled threshold picks
 * candidates in many workgroups per row, one workgroup per row selects among them, with a
 * whole-row select when the candidates cannot hold the answer). A path the shape does not
 * allow falls back to the automatic choice. key "score_chunks_per_wave": 64-key chunks
 * each wave of the 16-bit decode scoring kernel walks (0 = automatic, else 1..64, taken
 * down to 1, 2, 4 or 8). key "score_prefill_waves": waves per workgroup of the 16-bit
 * scoring kernel for 8 or more queries per sequence, each wave taking 2 queries (0 =
 * automatic, else 4 or 8). key "mla_tiles_per_step": 16-row tiles of selected latent rows
 * that the 16-bit sparse MLA kernel takes between two workgroup barriers (0 = automatic: 3
 * when a part holds at least 1024 selected slots, else 2; or 1, 2 or 3 for every call; all
 * give results within the same tolerance, with a different summation order). key
 * "mla_head_split": run each query's 64 heads as two 32-head workgroups sharing the query's
 * selected rows (0 = automatic: when 64-head workgroups would fill at most half of the 256
 * CUs; 1 = never; 2 = always for 64 heads). key "topk_cand_block": threads of the workgroup that
 * selects a row's top-k among the candidates of dsa_index_score_topk (0 = automatic (1024),
 * 256, 512 or 1024). Returns DSA_OK,
 * or DSA_ERR_SHAPE for an unknown key or value. The switches are process-wide state (atomic);
 * every call reads the ones it uses once, when it starts, so a change applies to later calls.
 */
int dsa_set_tuning(const char* key, int value);

/*
 * Pooled (kpool) indexer, a second DSA variant (vllm-rdna pull request "Glm5Next
 * (GLM-5.3-Flash) on gfx1030": architecture section, DSA attention commit and first-cut
 * kernel commit). The indexer cache keeps one packed row per token, k[D] | gate[D] | valid
 * (257 values for D = 128); groups of kpool consecutive tokens (pools) are compressed into
 * one key with softmax(gate + ape) weights, queries score pool keys, top-k picks pools, and
 * the attended set is the selected pools' tokens plus the last incomplete pool (the tail),
 * which is always attended. A decode step is dsa_kpool_index_score -> dsa_topk over pools
 * (top_pools = top_k / kpool) -> dsa_kpool_expand -> dsa_sparse_mla_attn over the tokens
 * (or dsa_kpool_sparse_mla_attn for the last two).
 */

/*
 * Pool keys of pools [pool_begin, pool_end) of every sequence:
 *
 *   pooled[b][p][d] = sum_j softmax_j(gate[t_j][d] + ape[j][d]) * k[t_j][d]
 *
 * over the pool's tokens t_j = kpool p + j (j < kpool) whose valid entry is nonzero (+0 and
 * -0 are not valid); a pool without valid tokens gets the zero key. Computed in fp32 and
 * rounded to out_dtype (nearest even).
 *
 * packed     device, [B][n_kv][row_stride] of row_dtype: k in columns 0..D-1, gate in
 *            D..2D-1, valid in column 2D (row_stride >= 2 D + 1; 257 packs D = 128 rows)
 * ape        device, [kpool][D] fp32 position embedding of a token's slot in its pool
 * pooled     device, [B][n_kv / kpool][D] of out_dtype (the pool cache); only the given
 *            pools are written
 * 1 <= kpool <= 8, D <= 4096, 0 <= pool_begin <= pool_end <= n_kv / kpool and
 * (pool_end - pool_begin) * D < 2^31 (a decode step compresses the one pool that its new
 * token completes; a prefill compresses them all).
 */
int dsa_kpool_compress(const void* packed, int row_stride, int row_dtype, const float* ape, void* pooled,
                       int out_dtype, int B, int n_kv, int D, int kpool, int pool_begin, int pool_end,
                       hipStream_t stream);

/*
 * Scores of pool keys: dsa_index_score over the pool cache (n_pool = pools per sequence),
 * with kv_len and q_pos in tokens. Pool p is scored when all its tokens are in the cache and
 * the last one is at or before the query: kpool (p + 1) <= kv_len[b] and
 * kpool p + kpool - 1 <= q_pos[b][i]; otherwise its score is -inf. Shapes, dtypes, defaults
 * (kv_len NULL: n_pool * kpool tokens; q_pos NULL: kv_len - n_q + i) and errors as in
 * dsa_index_score; scores is [B][n_q][n_pool]. 1 <= kpool <= 8.
 */
int dsa_kpool_index_score(const void* q, const void* pooled, const float* w, const int32_t* kv_len,
                          const int32_t* q_pos, float* scores, int B, int n_q, int H, int D, int n_pool,
                          int kpool, int q_dtype, int k_dtype, float scale, hipStream_t stream);

/*
 * Selected pools -> attended tokens.
 *
 *   tok_idx[b][i][kpool s + j]           = kpool * pool_idx[b][i][s] + j      (s < top_pools, j < kpool)
 *   tok_idx[b][i][kpool top_pools + j]   = kpool * floor((pos + 1) / kpool) + j   (j < kpool - 1, the tail)
 *
 * with -1 for a -1 pool, a token whose valid entry is zero, a token at or past kv_len[b], and
 * a tail token after the query position pos = q_pos[b][i]. The width is
 * kpool * top_pools + kpool - 1 (2051 for 512 pools of 4); pool order is kept, so ascending
 * pool indices (dsa_topk's output) give ascending tokens.
 *
 * pool_idx   device, [B][n_q][top_pools] int32 (dsa_topk over the pool scores)
 * packed     device, the packed rows of dsa_kpool_compress (only the valid column is read)
 * kv_len     device, [B] int32 tokens, or NULL (n_kv)
 * q_pos      device, [B][n_q] int32 token positions, or NULL (kv_len - n_q + i)
 * tok_idx    device, [B][n_q][kpool * top_pools + kpool - 1] int32 out
 * B * n_q <= 65535, 1 <= kpool <= 8.
 */
int dsa_kpool_expand(const int32_t* pool_idx, const void* packed, int row_stride, int row_dtype, int D,
                     const int32_t* kv_len, const int32_t* q_pos, int32_t* tok_idx, int B, int n_q, int n_kv,
                     int top_pools, int kpool, hipStream_t stream);

/* dsa_kpool_expand followed by dsa_sparse_mla_attn in one call: the attention kernel makes
 * each part's token indices from pool_idx itself (the same tokens, in the same slot order, as
 * tok_idx above), so the expanded index array is never written. Arguments as in the two calls
 * it replaces; top_k of the attention is kpool * top_pools + kpool - 1 (n_split and the
 * workspace size are taken for that top_k), and the latent cache and the packed rows share
 * n_kv and kv_len. Only the MFMA attention shapes (bf16, Hm a multiple of 16 up to 64,
 * d_latent 512, d_rope 0 or 64); others return DSA_ERR_UNSUPPORTED (use the two calls).
 * Results are bit-identical to dsa_kpool_expand + dsa_sparse_mla_attn with the same n_split. */
int dsa_kpool_sparse_mla_attn(const void* q_abs, const void* latent, const int32_t* pool_idx, const void* packed,
                              int row_stride, int row_dtype, int D, const int32_t* kv_len, const int32_t* q_pos,
                              float* out, float* lse, int B, int n_q, int Hm, int n_kv, int top_pools, int kpool,
                              int d_latent, int d_rope, float sm_scale, int dtype, int n_split, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Static text of a status code. */
const char* dsa_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* dsa_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_DSA_H */
