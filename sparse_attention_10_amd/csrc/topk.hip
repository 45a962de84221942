// Top-k selection over fp32 score rows (ik_llama_opt commit log, sub-commit "Add
// GLM-5.2/DeepSeek-V3.2 DSA lightning indexer": top_k of min(top_k, n_tokens), used as a set;
// sub-commit "decode-correct via persistent indexer-K cache": the CUDA bitonic argsort could not
// take more than 1024 columns and fell back to the CPU, which is why this is a radix select).
//
// Scores map to order-preserving uint32 keys (-0 -> +0; NaN and -inf -> 0, "not valid").
// A workgroup finds the K-th largest key T with three histogram rounds (bits 31..20, 19..8,
// 7..0) over its row, then writes every key > T plus the lowest-index keys == T in ascending
// index order: a wave-ballot compaction where each wave owns a contiguous range, so output
// positions come from popcounts and never from atomics. The result is unique, hence bitwise
// deterministic.
//
// Paths: one workgroup per row (rows up to 32768 entries live in LDS), or two stages for
// long rows / few rows: stage 1 selects the top-k of every segment, stage 2 selects the top-k
// of the concatenated candidates. A row's top-k lies inside the union of its segments'
// top-k sets, and candidates stay in ascending index order, so both paths give the same
// answer.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dsa {

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (!(f == f)) return 0u;          // NaN
  if (u == 0xff800000u) return 0u;   // -inf
  if (u == 0x80000000u) u = 0u;      // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the threads of the block (thread order); *total gets the sum.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wsum, uint32_t* total) {
  constexpr int NW = BLOCK / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t ws = s_wsum[w];
    before += w < wave ? ws : 0u;
    tot += ws;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// The bin d holding the need-th largest counted key: above(d) < need <= above(d) + hist[d],
// with above(d) the count of bins > d. Result in s_sel[0] = d, s_sel[1] = above(d).
template <int BLOCK>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, uint32_t need, uint32_t* s_wsum,
                                         uint32_t* s_sel, uint32_t* total_out) {
  const int per = nb >= BLOCK ? nb / BLOCK : 1;
  const int gi = BLOCK - 1 - (int)threadIdx.x;  // thread 0 owns the highest bins
  const int lo = gi * per;
  uint32_t gsum = 0;
  if (lo < nb)
    for (int j = 0; j < per; ++j) gsum += hist[lo + j];
  uint32_t total;
  const uint32_t above = block_exclusive_scan<BLOCK>(gsum, s_wsum, &total);
  if (lo < nb && above < need && need <= above + gsum) {
    uint32_t acc = above;
    for (int j = per - 1; j >= 0; --j) {
      const uint32_t c = hist[lo + j];
      if (acc + c >= need) {
        s_sel[0] = (uint32_t)(lo + j);
        s_sel[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  *total_out = total;
}

// One workgroup per (segment, row). MAXN > 0 keeps the segment's keys in LDS; MAXN == 0 reads
// them from global memory on every pass (any length).
template <int BLOCK, int MAXN>
__global__ __launch_bounds__(BLOCK) void topk_rows(const float* __restrict__ vals, long row_stride,
                                                   int seg_len, int n_total,
                                                   const int* __restrict__ cand, int top_k,
                                                   int* __restrict__ out_idx,
                                                   float* __restrict__ out_val) {
  constexpr int NW = BLOCK / 64;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_keys[MAXN > 0 ? MAXN : 1];
  __shared__ uint32_t s_wsum[NW];
  __shared__ uint32_t s_wa[NW], s_wb[NW];
  __shared__ uint32_t s_sel[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y, seg = blockIdx.x;
  const long base = (long)row * row_stride + (long)seg * seg_len;
  const int n = min(seg_len, n_total - seg * seg_len);
  const int idx_base = seg * seg_len;
  const long obase = ((long)row * gridDim.x + seg) * top_k;
  int* o_idx = out_idx + obase;
  float* o_val = out_val ? out_val + obase : nullptr;

  auto key_at = [&](int e) -> uint32_t {
    if constexpr (MAXN > 0) return s_keys[e];
    else return score_key(vals[base + e]);
  };

  // round 0: load keys (into LDS) and count bits 31..20
  for (int j = tid; j < 4096; j += BLOCK) hist[j] = 0u;
  __syncthreads();
  for (int e = tid; e < n; e += BLOCK) {
    const uint32_t kk = score_key(vals[base + e]);
    if constexpr (MAXN > 0) s_keys[e] = kk;
    if (kk) atomicAdd(&hist[kk >> 20], 1u);
  }
  __syncthreads();

  uint32_t n_valid;
  // K is only known after the total; find_bin with need = top_k, then clamp.
  find_bin<BLOCK>(hist, 4096, (uint32_t)top_k, s_wsum, s_sel, &n_valid);
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) {
      o_idx[p] = -1;
      if (o_val) o_val[p] = -INFINITY;
    }
    return;
  }
  uint32_t need = K;
  uint32_t prefix, mask;
  if (K == (uint32_t)top_k) {
    prefix = s_sel[0] << 20;
    need -= s_sel[1];
  } else {
    // every valid key is taken: the threshold is the smallest valid key's bin
    __syncthreads();
    find_bin<BLOCK>(hist, 4096, K, s_wsum, s_sel, &n_valid);
    prefix = s_sel[0] << 20;
    need -= s_sel[1];
  }
  mask = 0xfff00000u;

  // round 1: bits 19..8 of the keys in bin prefix
  __syncthreads();
  for (int j = tid; j < 4096; j += BLOCK) hist[j] = 0u;
  __syncthreads();
  for (int e = tid; e < n; e += BLOCK) {
    const uint32_t kk = key_at(e);
    if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  uint32_t tmp;
  find_bin<BLOCK>(hist, 4096, need, s_wsum, s_sel, &tmp);
  prefix |= s_sel[0] << 8;
  need -= s_sel[1];
  mask = 0xffffff00u;

  // round 2: bits 7..0
  __syncthreads();
  for (int j = tid; j < 256; j += BLOCK) hist[j] = 0u;
  __syncthreads();
  for (int e = tid; e < n; e += BLOCK) {
    const uint32_t kk = key_at(e);
    if ((kk & mask) == prefix) atomicAdd(&hist[kk & 0xffu], 1u);
  }
  __syncthreads();
  find_bin<BLOCK>(hist, 256, need, s_wsum, s_sel, &tmp);
  const uint32_t T = prefix | s_sel[0];
  need -= s_sel[1];  // keys == T still to take, lowest index first (>= 1)

  // ordered compaction: wave w owns the 64-wide steps [w * spw, (w + 1) * spw)
  const int steps = (n + 63) / 64;
  const int spw = (steps + NW - 1) / NW;
  const int st0 = wave * spw, st1 = min(steps, st0 + spw);
  uint32_t cgt = 0, ceq = 0;
  for (int st = st0; st < st1; ++st) {
    const int e = st * 64 + lane;
    const uint32_t kk = e < n ? key_at(e) : 0u;
    cgt += __popcll(__ballot(kk > T));
    ceq += __popcll(__ballot(kk == T));
  }
  if (lane == 0) {
    s_wa[wave] = cgt;
    s_wb[wave] = ceq;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t eqw = s_wb[w];
    const uint32_t take = need > eq_before ? min(eqw, need - eq_before) : 0u;
    sel_before += s_wa[w] + take;
    eq_before += eqw;
  }
  uint32_t run_eq = eq_before, run_sel = sel_before;
  for (int st = st0; st < st1; ++st) {
    const int e = st * 64 + lane;
    const uint32_t kk = e < n ? key_at(e) : 0u;
    const bool gt = kk > T;
    const bool eq = kk == T;
    const uint64_t beq = __ballot(eq);
    const bool sel = gt || (eq && run_eq + mbcnt(beq) < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t p = run_sel + mbcnt(bsel);
    if (sel && p < K) {
      o_idx[p] = cand ? cand[base + e] : idx_base + e;
      if (o_val) o_val[p] = key_value(kk);
    }
    run_eq += __popcll(beq);
    run_sel += __popcll(bsel);
  }
  for (int p = (int)K + tid; p < top_k; p += BLOCK) {
    o_idx[p] = -1;
    if (o_val) o_val[p] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static constexpr int kResidentMax = 32768;
static constexpr int kSegTarget = 8192;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

TopkPlan plan_topk(int rows, int n_kv, int top_k, int path) {
  TopkPlan p{0, 1, n_kv, 0};
  // two-stage feasibility: segments shorter than the row, each keeps top_k candidates, and
  // the candidates of a row fit one LDS-resident stage-2 pass
  int S = (n_kv + kSegTarget - 1) / kSegTarget;
  if (S < 2) S = 2;
  int seg = (n_kv + S - 1) / S;
  seg = (seg + 63) / 64 * 64;
  S = (n_kv + seg - 1) / seg;
  const bool feasible = S >= 2 && (long)S * top_k <= kResidentMax && seg <= kResidentMax &&
                        seg >= 2 * top_k;
  bool use = false;
  if (path == 2) use = feasible;
  else if (path == 0) use = feasible && (n_kv > kResidentMax || (rows < 128 && n_kv >= 4 * top_k));
  if (feasible) {
    const size_t cand = (size_t)rows * S * top_k;
    p.ws_bytes = align256(cand * sizeof(int)) + align256(cand * sizeof(float));
  }
  if (use) {
    p.two_stage = 1;
    p.segments = S;
    p.seg_len = seg;
  }
  return p;
}

static void launch_rows(const float* vals, long row_stride, int seg_len, int n_total, int S, int rows,
                        const int* cand, int top_k, int* out_idx, float* out_val, hipStream_t stream) {
  const int n = seg_len;  // longest segment
  dim3 grid(S, rows);
  if (n <= 2048)
    hipLaunchKernelGGL((topk_rows<256, 2048>), grid, dim3(256), 0, stream, vals, row_stride, seg_len,
                       n_total, cand, top_k, out_idx, out_val);
  else if (n <= 8192)
    hipLaunchKernelGGL((topk_rows<512, 8192>), grid, dim3(512), 0, stream, vals, row_stride, seg_len,
                       n_total, cand, top_k, out_idx, out_val);
  else if (n <= kResidentMax)
    hipLaunchKernelGGL((topk_rows<1024, kResidentMax>), grid, dim3(1024), 0, stream, vals, row_stride,
                       seg_len, n_total, cand, top_k, out_idx, out_val);
  else
    hipLaunchKernelGGL((topk_rows<1024, 0>), grid, dim3(1024), 0, stream, vals, row_stride, seg_len,
                       n_total, cand, top_k, out_idx, out_val);
}

hipError_t launch_topk(const float* scores, int* idx, int rows, int n_kv, int top_k,
                       const TopkPlan& plan, void* workspace, hipStream_t stream) {
  if (!plan.two_stage) {
    launch_rows(scores, n_kv, n_kv, n_kv, 1, rows, nullptr, top_k, idx, nullptr, stream);
    return hipGetLastError();
  }
  const size_t cand = (size_t)rows * plan.segments * top_k;
  int* ws_idx = reinterpret_cast<int*>(workspace);
  float* ws_val = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(cand * sizeof(int)));
  launch_rows(scores, n_kv, plan.seg_len, n_kv, plan.segments, rows, nullptr, top_k, ws_idx, ws_val, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int m = plan.segments * top_k;
  launch_rows(ws_val, m, m, m, 1, rows, ws_idx, top_k, idx, nullptr, stream);
  return hipGetLastError();
}

}  // namespace dsa
