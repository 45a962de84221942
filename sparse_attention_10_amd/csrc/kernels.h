// Launchers of the libdsa kernels (internal; the public interface is include/dsa.h).
// Each launcher assumes validated arguments and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>
#include <stdint.h>

namespace dsa {

constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;

// Score options. Attention-sink boost: scores of keys [start[b], start[b] + n) of sequence b
// get + boost (start NULL: 0; n = 0: off); masked keys stay -inf. kpool: each key stands for a
// pool of kpool consecutive tokens, while kv_len and q_pos stay in tokens (1: keys are tokens).
struct ScoreArgs {
  const int* start;
  int n;
  float boost;
  int kpool;
};

// Tuning switches (dsa_set_tuning): process-wide, each read once per call.
// Candidate output of the decode score kernel for the fused score -> top-k call: every wave
// (n_w per row, each over its own G = ITERS * 64 consecutive keys) writes min(valid, m) of its
// valid keys (order-preserving keys) in index order as (key, index) pairs, key 0 in the slots
// it leaves unused, and a header {kept, valid keys, bound tau, 0}: when it holds more than m
// valid keys, every key it did not keep is at most tau (else tau = 0).
struct CandOut {
  uint2* kv;   // [rows][n_w * m]: (key, index) pairs, 8 bytes each
  uint4* hdr;  // [rows][n_w]
  int m;
};
// Plan of the fused score -> top-k path for decode rows (16-bit, D = 128, H <= 32, n_q < 8):
// chunks per wave, candidates per wave, waves per row; ok = false when the shape is not one
// the fused kernels take (then the call runs the score and top-k kernels one after the other).
struct ScoreTopkPlan {
  bool ok;
  int iters, m, n_w;
  size_t cand_bytes;  // candidate keys, indices and headers
  bool wide;          // more than kCandCap candidates per row: the select holds kCandCapWide
};
constexpr int kCandCap = 8192;        // candidates one select workgroup holds in registers
constexpr int kCandCapWide = 16384;   // the same with 16 per thread, for rows of more ranges
constexpr int kCandMaxWaves = 1024;  // candidate ranges (waves) per row
extern std::atomic<int> g_topk_cand_block;  // threads of the candidate select workgroup (0: 1024)
ScoreTopkPlan plan_score_topk(int B, int n_q, int H, int D, int n_kv, int top_k, int dtype);
hipError_t launch_index_score_cand(const void* q, const void* k, const float* w, const int* kv_len,
                                   const int* q_pos, float* scores, int B, int n_q, int H, int n_kv, int dtype,
                                   float scale, const ScoreTopkPlan& plan, CandOut cand, hipStream_t stream);
hipError_t launch_topk_cand(const float* scores, int* idx, int rows, int n_kv, int top_k,
                            const ScoreTopkPlan& plan, const CandOut& cand, hipStream_t stream);

extern std::atomic<int> g_score_cpw;            // 64-key chunks per wave of the decode scoring kernel, 0 automatic
extern std::atomic<int> g_score_prefill_waves;  // waves per block of the prefill scoring kernel (4 or 8), 0 automatic
hipError_t launch_index_score(const void* q, const void* k, const float* w, const int* kv_len,
                              const int* q_pos, float* scores, int B, int n_q, int H, int D,
                              int n_kv, int dtype, float scale, ScoreArgs sink, hipStream_t stream);

// top-k: path 0 = automatic, 1 = one workgroup per row, 2 = two-stage, 3 = filtered
struct TopkPlan {
  int kind;        // 0 one workgroup per row, 1 two-stage (segments + candidates), 2 filtered
  int segments;    // segments per row (two-stage, filtered)
  int seg_len;     // elements per segment (two-stage, filtered)
  uint32_t need;   // filtered: sampled keys the threshold must cover
  size_t ws_bytes; // workspace any path of this shape may use
};
TopkPlan plan_topk(int rows, int n_kv, int top_k, int path);
hipError_t launch_topk(const float* scores, int* idx, int rows, int n_kv, int top_k,
                       const TopkPlan& plan, void* workspace, hipStream_t stream);
// the static top-k scratch of the current device (its device address; looked up once per device)
constexpr size_t kTopkScratchBytes = size_t(16) << 20;
hipError_t topk_scratch(void** ptr);

// sparse MLA
extern std::atomic<int> g_mla_tiles_per_step;  // 16-row tiles per step of the 16-bit MLA kernel (0 automatic, 1, 2 or 3)
extern std::atomic<int> g_mla_head_split;      // 64 heads as two 32-head workgroup rows: 0 automatic, 1 never, 2 always
int mla_auto_splits(int B, int n_q, int top_k);
size_t mla_workspace_bytes(int B, int n_q, int Hm, int top_k, int d_latent, int n_split);
bool mla_mfma_supported(int Hm, int d_latent, int d_rope, int dtype);
// Slot indices of the pooled indexer, made by the attention kernel itself while it stages
// a part's slots: slot s < kpool * top_pools is token kpool * pool_idx[s / kpool] + s % kpool,
// the last kpool - 1 slots are the tail kpool * floor((pos + 1) / kpool) .. pos; a token is
// kept only if it is in the cache and its packed row's valid entry is nonzero (the same rule
// as launch_kpool_expand). top_k of the attention is then kpool * top_pools + kpool - 1.
struct KpoolSlots {
  const int* pool_idx;    // [B * n_q][top_pools]
  const uint8_t* packed;  // packed k | gate | valid rows, [B][n_kv]
  long row_bytes;         // bytes per packed row
  int valid_off;          // byte offset of the valid entry in a row
  int valid_f32;          // 1: the valid entry is fp32, else 16-bit
  int top_pools;
  int kpool;
  const int* q_pos;       // [B * n_q] or null (query i of a sequence at len - n_q + i)
};
hipError_t launch_sparse_mla(const void* q_abs, const void* latent, const int* idx,
                             const int* kv_len, float* out, float* lse, int B, int n_q, int Hm,
                             int n_kv, int top_k, int d_latent, int d_rope, float sm_scale,
                             int dtype, int n_split, void* workspace, hipStream_t stream,
                             const KpoolSlots* kp = nullptr);  // kp: MFMA shapes only, idx unused

// indexer-input preparation (rope + Hadamard + cache append)
hipError_t launch_indexer_prep(const float* q_in, const float* k_in, const void* latent_in, const int* pos,
                               void* q_out, void* k_cache, void* latent_cache, int B, int n_new, int H,
                               int n_kv, int row_bytes, int out_dtype, double log2_base, int hadamard,
                               hipStream_t stream);

// pooled indexer: pool compression of packed k | gate | valid rows, pool -> token expansion
hipError_t launch_kpool_compress(const void* packed, int row_stride, int row_dtype, const float* ape,
                                 void* pooled, int out_dtype, int B, int n_kv, int D, int kpool,
                                 int pool_begin, int pool_end, hipStream_t stream);
hipError_t launch_kpool_expand(const int* pool_idx, const void* packed, int row_stride, int row_dtype, int D,
                               const int* kv_len, const int* q_pos, int* tok_idx, int B, int n_q, int n_kv,
                               int top_pools, int kpool, hipStream_t stream);

}  // namespace dsa
