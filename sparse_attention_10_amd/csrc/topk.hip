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
                                         uint32_t* s_sel) {
  const int per = (nb + BLOCK - 1) / BLOCK;
  const int gi = BLOCK - 1 - (int)threadIdx.x;  // thread 0 owns the highest bins
  const int lo = gi * per;
  const int hi = min(nb, lo + per);
  uint32_t gsum = 0;
  for (int j = lo; j < hi; ++j) gsum += hist[j];
  uint32_t total;
  const uint32_t above = block_exclusive_scan<BLOCK>(gsum, s_wsum, &total);
  if (lo < hi && above < need && need <= above + gsum) {
    uint32_t acc = above;
    for (int j = hi - 1; j >= lo; --j) {
      const uint32_t c = hist[j];
      if (acc + c >= need) {
        s_sel[0] = (uint32_t)j;
        s_sel[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int bit_width(uint32_t x) { return x ? 32 - __clz(x) : 0; }

// Streaming fallback for segments longer than the register-resident kernels take: one
// workgroup per (segment, row); MAXN > 0 would keep keys in LDS, MAXN == 0 reads them from
// global memory on every pass (any length).
//
// Radix rounds on a shrinking key range [lo, lo + span]: each round bins (key - lo) >> shift
// into at most 4096 bins with shift = max(0, bit_width(span) - 12), picks the bin holding the
// need-th largest key and narrows the range to it. The first range is [min, max] of the row's
// valid keys, so the bins cover where the scores actually are (scores of one row usually sit
// within a binade or two; fixed top-bit digits would pile them into a few bins and serialise
// the LDS atomics). At most three rounds reach shift 0, where lo is the K-th largest key.
template <int BLOCK, int MAXN, bool CAND>
__global__ __launch_bounds__(BLOCK) void topk_rows(const float* __restrict__ vals, long row_stride,
                                                   int seg_len, int n_total,
                                                   const int* __restrict__ cand, int top_k,
                                                   int* __restrict__ out_idx,
                                                   float* __restrict__ out_val) {
  constexpr int NW = BLOCK / 64;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t s_keys[MAXN > 0 ? MAXN : 1];
  __shared__ int s_cand[(MAXN > 0 && CAND) ? MAXN : 1];  // candidate indices (stage 2)
  __shared__ uint32_t s_wsum[NW];
  __shared__ uint32_t s_wa[NW], s_wb[NW], s_wc[NW];
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

  // pass 0: keys into LDS; count, min and max of the valid keys. The loads of a batch are
  // issued together (unrolled) so their memory latencies overlap.
  constexpr int ITEMS = MAXN > 0 ? MAXN / BLOCK : 8;
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
  for (int e0 = 0; e0 < n; e0 += ITEMS * BLOCK) {
    float v[ITEMS];
    int ci[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = e0 + j * BLOCK + tid;
      v[j] = e < n ? vals[base + e] : __int_as_float(0x7fc00000);
      if constexpr (CAND && MAXN > 0) ci[j] = e < n ? cand[base + e] : -1;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = e0 + j * BLOCK + tid;
      const uint32_t kk = score_key(v[j]);
      if constexpr (MAXN > 0) {
        if (e < n) s_keys[e] = kk;
        if constexpr (CAND) {
          if (e < n) s_cand[e] = ci[j];
        }
      }
      if (kk) {
        ++cnt;
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, off, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, off, 64));
  }
  if (lane == 0) {
    s_wa[wave] = cnt;
    s_wb[wave] = kmin;
    s_wc[wave] = kmax;
  }
  __syncthreads();
  uint32_t n_valid = 0;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_valid += s_wa[w];
    kmin = min(kmin, s_wb[w]);
    kmax = max(kmax, s_wc[w]);
  }
  __syncthreads();
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) {
      o_idx[p] = -1;
      if (o_val) o_val[p] = -INFINITY;
    }
    return;
  }

  uint32_t need = K;
  uint32_t lo = kmin, span = kmax - kmin;
  for (int round = 0; round < 4; ++round) {
    const int shift = max(0, bit_width(span) - 12);
    const int nb = (int)(span >> shift) + 1;
    for (int j = tid; j < nb; j += BLOCK) hist[j] = 0u;
    __syncthreads();
    for (int e = tid; e < n; e += BLOCK) {
      const uint32_t kk = key_at(e);
      const uint32_t rel = kk - lo;
      if (kk && kk >= lo && rel <= span) atomicAdd(&hist[rel >> shift], 1u);
    }
    __syncthreads();
    find_bin<BLOCK>(hist, nb, need, s_wsum, s_sel);
    const uint32_t d = s_sel[0];
    need -= s_sel[1];
    lo += d << shift;
    if (shift == 0) break;
    span = min(span - (d << shift), (1u << shift) - 1u);
    __syncthreads();
  }
  const uint32_t T = lo;  // the K-th largest key; `need` keys equal to T are taken (>= 1)

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
      int ix = idx_base + e;
      if constexpr (CAND) {
        if constexpr (MAXN > 0) ix = s_cand[e];
        else ix = cand[base + e];
      }
      o_idx[p] = ix;
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
// Register-resident kernel: thread t holds elements j * BLOCK + t (j < ITEMS) of its segment,
// so a wave's lanes hold 64 consecutive elements for each j ("chunk" j * NW + wave, chunks in
// ascending element order). Histogram rounds read keys from registers and issue their LDS
// atomics back to back; 8192 bins usually finish in two rounds. The ordered compaction
// counts every chunk's keys > T and == T with ballots, turns the counts into output offsets
// with two block scans, and writes each chunk with ballot + mbcnt.
// ---------------------------------------------------------------------------------------
template <int BLOCK, int ITEMS, bool CAND>
__global__ __launch_bounds__(BLOCK) void topk_rows_reg(const float* __restrict__ vals, long row_stride,
                                                       int seg_len, int n_total,
                                                       const int* __restrict__ cand, int top_k,
                                                       int* __restrict__ out_idx,
                                                       float* __restrict__ out_val) {
  constexpr int NW = BLOCK / 64;
  constexpr int NB = 8192;
  constexpr int NCH = ITEMS * NW;  // chunks of 64
  static_assert(NCH <= BLOCK, "one thread per chunk in the offset scans");
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t s_wsum[NW];
  __shared__ uint32_t s_wa[NW], s_wb[NW], s_wc[NW];
  __shared__ uint32_t s_gt[NCH], s_eq[NCH];
  __shared__ uint32_t s_sel[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y, seg = blockIdx.x;
  const long base = (long)row * row_stride + (long)seg * seg_len;
  const int n = min(seg_len, n_total - seg * seg_len);
  const int idx_base = seg * seg_len;
  const long obase = ((long)row * gridDim.x + seg) * top_k;
  int* o_idx = out_idx + obase;
  float* o_val = out_val ? out_val + obase : nullptr;

  uint32_t key[ITEMS];
  int ci[ITEMS];
  {
    float v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = j * BLOCK + tid;
      v[j] = e < n ? vals[base + e] : __int_as_float(0x7fc00000);
      if constexpr (CAND) ci[j] = e < n ? cand[base + e] : -1;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) key[j] = score_key(v[j]);
  }
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    if (key[j]) {
      ++cnt;
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, off, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, off, 64));
  }
  if (lane == 0) {
    s_wa[wave] = cnt;
    s_wb[wave] = kmin;
    s_wc[wave] = kmax;
  }
  __syncthreads();
  uint32_t n_valid = 0;
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_valid += s_wa[w];
    kmin = min(kmin, s_wb[w]);
    kmax = max(kmax, s_wc[w]);
  }
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) {
      o_idx[p] = -1;
      if (o_val) o_val[p] = -INFINITY;
    }
    return;
  }

  // radix rounds on the shrinking key range [lo, lo + span]
  uint32_t need = K;
  uint32_t lo = kmin, span = kmax - kmin;
  for (int round = 0; round < 4; ++round) {
    const int shift = max(0, bit_width(span) - 13);
    const int nb = (int)(span >> shift) + 1;
    for (int j = tid; j < nb; j += BLOCK) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t rel = key[j] - lo;
      if (key[j] && key[j] >= lo && rel <= span) atomicAdd(&hist[rel >> shift], 1u);
    }
    __syncthreads();
    find_bin<BLOCK>(hist, nb, need, s_wsum, s_sel);
    const uint32_t d = s_sel[0];
    need -= s_sel[1];
    lo += d << shift;
    if (shift == 0) break;
    span = min(span - (d << shift), (1u << shift) - 1u);
    __syncthreads();
  }
  const uint32_t T = lo;  // the K-th largest key; `need` keys equal to T are taken (>= 1)

  // per-chunk counts
  uint64_t bgt[ITEMS], beq[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    bgt[j] = __ballot(key[j] > T);
    beq[j] = __ballot(key[j] == T);
    if (lane == 0) {
      s_gt[j * NW + wave] = (uint32_t)__popcll(bgt[j]);
      s_eq[j * NW + wave] = (uint32_t)__popcll(beq[j]);
    }
  }
  __syncthreads();
  // chunk c = tid: keys == T before it, then output offset before it
  const uint32_t my_eq = tid < NCH ? s_eq[tid] : 0u;
  const uint32_t my_gt = tid < NCH ? s_gt[tid] : 0u;
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan<BLOCK>(my_eq, s_wsum, &tot);
  const uint32_t take = need > eq_before ? min(my_eq, need - eq_before) : 0u;
  const uint32_t sel_before = block_exclusive_scan<BLOCK>(my_gt + take, s_wsum, &tot);
  if (tid < NCH) {
    s_eq[tid] = eq_before;
    s_gt[tid] = sel_before;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int c = j * NW + wave;
    const uint32_t eqb = s_eq[c], selb = s_gt[c];
    const bool gt = key[j] > T;
    const bool eq = key[j] == T;
    const bool sel = gt || (eq && eqb + mbcnt(beq[j]) < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t p = selb + mbcnt(bsel);
    if (sel && p < K) {
      int ix = idx_base + j * BLOCK + tid;
      if constexpr (CAND) ix = ci[j];
      o_idx[p] = ix;
      if (o_val) o_val[p] = key_value(key[j]);
    }
  }
  for (int p = (int)K + tid; p < top_k; p += BLOCK) {
    o_idx[p] = -1;
    if (o_val) o_val[p] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static constexpr int kResidentMax = 32768;  // longest segment held in registers by one workgroup
static constexpr int kCandMax = 32768;      // candidates of one row in the second stage
static constexpr int kSegTarget = 8192;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

TopkPlan plan_topk(int rows, int n_kv, int top_k, int path) {
  TopkPlan p{0, 1, n_kv, 0};
  // two-stage feasibility: segments shorter than the row, each keeps top_k candidates, and
  // the candidates of a row fit one LDS-resident stage-2 pass
  // segments of about kSegTarget entries, but no more candidates than one LDS-resident
  // stage-2 pass with indices holds
  int S = (n_kv + kSegTarget - 1) / kSegTarget;
  if (S > kCandMax / top_k) S = kCandMax / top_k;
  if (S < 2) S = 2;
  int seg = (n_kv + S - 1) / S;
  seg = (seg + 63) / 64 * 64;
  S = (n_kv + seg - 1) / seg;
  const bool feasible = S >= 2 && (long)S * top_k <= kCandMax && seg <= kResidentMax && seg >= 2 * top_k;
  bool use = false;
  if (path == 2) use = feasible;
  else if (path == 0) use = feasible && n_kv > kResidentMax;  // one pass is faster when it fits
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

template <bool CAND>
static void launch_rows_t(const float* vals, long row_stride, int seg_len, int n_total, int S, int rows,
                          const int* cand, int top_k, int* out_idx, float* out_val, hipStream_t stream) {
  const int n = seg_len;  // longest segment
  dim3 grid(S, rows);
#define DSA_TOPK_REG(BL, IT)                                                                      \
  hipLaunchKernelGGL((topk_rows_reg<BL, IT, CAND>), grid, dim3(BL), 0, stream, vals, row_stride, \
                     seg_len, n_total, cand, top_k, out_idx, out_val)
  if (n <= 256 * 8) DSA_TOPK_REG(256, 8);
  else if (n <= 512 * 16) DSA_TOPK_REG(512, 16);
  else if (n <= 512 * 32) DSA_TOPK_REG(512, 32);
  else if (n <= 1024 * 32) DSA_TOPK_REG(1024, 32);
  else
    hipLaunchKernelGGL((topk_rows<1024, 0, CAND>), grid, dim3(1024), 0, stream, vals, row_stride, seg_len,
                       n_total, cand, top_k, out_idx, out_val);
#undef DSA_TOPK_REG
}

static void launch_rows(const float* vals, long row_stride, int seg_len, int n_total, int S, int rows,
                        const int* cand, int top_k, int* out_idx, float* out_val, hipStream_t stream) {
  if (cand)
    launch_rows_t<true>(vals, row_stride, seg_len, n_total, S, rows, cand, top_k, out_idx, out_val, stream);
  else
    launch_rows_t<false>(vals, row_stride, seg_len, n_total, S, rows, cand, top_k, out_idx, out_val, stream);
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
