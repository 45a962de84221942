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
// Paths (all give the same unique result):
//  - one workgroup per row, keys in registers (rows up to 32768 entries; longer rows stream);
//  - two-stage for long rows: stage 1 selects the top-k of every segment, stage 2 the top-k
//    of the concatenated candidates. A row's top-k lies inside the union of its segments'
//    top-k sets, and candidates stay in ascending index order;
//  - filtered, for few rows: many workgroups per row keep only the keys at or above a
//    threshold taken from a sample of the row, then one workgroup per row selects among
//    them, or from the whole row when the threshold was too high.
#include "common.h"
#include "kernels.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

namespace dsa {

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
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

// Wave-wide inclusive scans in DPP (no LDS round trips): row_shr 1, 2, 4, 8 scan each
// 16-lane row, then the last lane of rows 0 and 2 is broadcast into rows 1 and 3 and lane
// 31 into rows 2 and 3. Lanes without a source take the operation's identity.
#define DSA_DPP(id, x, ctrl, rows) \
  ((uint32_t)__builtin_amdgcn_update_dpp((int)(id), (int)(x), (ctrl), (rows), 0xf, false))
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, DSA_DPP(id, x, 0x111, 0xf));
  x = op(x, DSA_DPP(id, x, 0x112, 0xf));
  x = op(x, DSA_DPP(id, x, 0x114, 0xf));
  x = op(x, DSA_DPP(id, x, 0x118, 0xf));
  x = op(x, DSA_DPP(id, x, 0x142, 0xa));
  x = op(x, DSA_DPP(id, x, 0x143, 0xc));
  return x;
}
#undef DSA_DPP
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); } };

__device__ __forceinline__ uint32_t lane_value(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}
// sums from lane 0 up to this lane
__device__ __forceinline__ uint32_t wave_scan_up(uint32_t x) { return wave_scan(x, 0u, OpAdd()); }
// sums from this lane up to lane 63
__device__ __forceinline__ uint32_t wave_scan_down(uint32_t x) {
  const uint32_t incl = wave_scan_up(x);
  return lane_value(incl, 63) - incl + x;
}
// count, min and max over the wave, the same in every lane
__device__ __forceinline__ void wave_count_min_max(uint32_t& cnt, uint32_t& kmin, uint32_t& kmax) {
  cnt = lane_value(wave_scan(cnt, 0u, OpAdd()), 63);
  kmin = lane_value(wave_scan(kmin, 0xffffffffu, OpMin()), 63);
  kmax = lane_value(wave_scan(kmax, 0u, OpMax()), 63);
}
// count, min, max and a second sum over the workgroup, the same in every thread. Each wave
// reduces its lanes and leaves (count, min, max, sum) in red[wave]; wave 0 reduces those and
// leaves the totals in red[BLOCK / 64], which every thread then reads once (rather than every
// thread reading every wave's entry). red holds BLOCK / 64 + 1 entries.
template <int BLOCK>
__device__ __forceinline__ void block_count_min_max(uint32_t& cnt, uint32_t& kmin, uint32_t& kmax, uint32_t& sum,
                                                    uint4* red) {
  constexpr int NW = BLOCK / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_count_min_max(cnt, kmin, kmax);
  sum = lane_value(wave_scan(sum, 0u, OpAdd()), 63);
  if (lane == 0) red[wave] = make_uint4(cnt, kmin, kmax, sum);
  __syncthreads();
  if (wave == 0) {
    const uint4 r = lane < NW ? red[lane] : make_uint4(0u, 0xffffffffu, 0u, 0u);
    uint32_t c = r.x, mn = r.y, mx = r.z;
    wave_count_min_max(c, mn, mx);
    const uint32_t sw = lane_value(wave_scan((uint32_t)r.w, 0u, OpAdd()), 63);
    if (lane == 0) red[NW] = make_uint4(c, mn, mx, sw);
  }
  __syncthreads();
  const uint4 t = red[NW];
  cnt = t.x;
  kmin = t.y;
  kmax = t.z;
  sum = t.w;
}

// Finding the bin d of hist[0, NB) (bins ascend with the key) that holds the need-th largest
// counted key, 1 <= need <= total count: the workgroup sums runs of bins (bin_parts), one
// wave gives lane l the count of bins [l * PL, (l + 1) * PL) and its suffix sum
// (wave_part_scan), and the lane whose range holds the target has its range split over the
// wave again (wave_find_in).
struct BinScan {
  uint32_t sum;   // keys in this lane's bins
  uint32_t incl;  // keys in this lane's bins and every bin above them
};

// First level, shared by the whole workgroup: part[t] = keys in bins [t * PT, (t + 1) * PT)
// with PT = NB / BLOCK (16-byte reads, each thread starting at a different slot of its
// range so that neighbouring threads hit different banks).
template <int BLOCK, int NB>
__device__ __forceinline__ void bin_parts(const uint32_t* hist, uint32_t* part) {
  constexpr int PT = NB / BLOCK, NR = PT / 4;
  static_assert(PT % 4 == 0, "16-byte reads");
  const int t = threadIdx.x;
  const uint4* h4 = reinterpret_cast<const uint4*>(hist + t * PT);
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const uint4 v = h4[(i + t) & (NR - 1)];
    s += v.x + v.y + v.z + v.w;
  }
  part[t] = s;
}

// Lane l of the calling wave: keys in bins [l * NB / 64, (l + 1) * NB / 64) from the parts.
template <int BLOCK, int NB>
__device__ __forceinline__ BinScan wave_part_scan(const uint32_t* part) {
  constexpr int PPL = BLOCK / 64;
  static_assert(PPL % 4 == 0, "16-byte reads");
  const int lane = threadIdx.x & 63;
  const uint4* p4 = reinterpret_cast<const uint4*>(part + lane * PPL);
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PPL / 4; ++i) {
    const uint4 v = p4[i];
    sum += v.x + v.y + v.z + v.w;
  }
  return BinScan{sum, wave_scan_down(sum)};
}

// Writes sel[0] = d, sel[1] = keys in bins above d, sel[2] = keys in bin d.
template <int NB>
__device__ __forceinline__ void wave_find_in(const uint32_t* hist, BinScan bs, uint32_t need, uint32_t* sel) {
  constexpr int PL = NB / 64, P2 = PL / 64;
  const int lane = threadIdx.x & 63;
  const uint64_t hit = __ballot(bs.incl - bs.sum < need && need <= bs.incl);
  const int f = __ffsll((unsigned long long)hit) - 1;
  const uint32_t above_f = lane_value(bs.incl - bs.sum, f);
  const int b0 = f * PL + lane * P2;
  uint32_t b[P2], s2 = 0;
#pragma unroll
  for (int k = 0; k < P2; ++k) {
    b[k] = hist[b0 + k];
    s2 += b[k];
  }
  const uint32_t a2 = above_f + wave_scan_down(s2) - s2;  // keys above this lane's bins
  if (a2 < need && need <= a2 + s2) {
    uint32_t acc = a2;
#pragma unroll
    for (int k = P2 - 1; k >= 0; --k) {
      if (acc < need && need <= acc + b[k]) {
        sel[0] = (uint32_t)(b0 + k);
        sel[1] = acc;
        sel[2] = b[k];
      }
      acc += b[k];
    }
  }
}


// ---------------------------------------------------------------------------------------
// Streaming select, any length: one workgroup reads its row from global memory on every
// pass. Radix rounds on a shrinking key range [lo, lo + span]: each round bins
// (key - lo) >> shift into at most 4096 bins with shift = max(0, bit_width(span) - 12), picks
// the bin holding the need-th largest key and narrows the range to it. The first range is
// [min, max] of the row's valid keys, so the bins cover where the scores actually are
// (scores of one row usually sit within a binade or two; fixed top-bit digits would pile
// them into a few bins and serialise the LDS atomics). At most three rounds reach shift 0,
// where lo is the K-th largest key.
// ---------------------------------------------------------------------------------------
template <int BLOCK>
struct StreamSmem {
  uint32_t hist[4096];
  uint4 red[BLOCK / 64 + 1];
  uint32_t wsum[BLOCK / 64], wa[BLOCK / 64], wb[BLOCK / 64];
  uint32_t sel[2];
};

template <int BLOCK>
__device__ __forceinline__ void select_streaming(StreamSmem<BLOCK>& sm, const float* __restrict__ vals, int n, int top_k,
                                 int* __restrict__ o_idx) {
  constexpr int NW = BLOCK / 64;
  constexpr int ITEMS = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // count, min and max of the valid keys; the loads of a batch are issued together
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
  for (int e0 = 0; e0 < n; e0 += ITEMS * BLOCK) {
    float v[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = e0 + j * BLOCK + tid;
      v[j] = e < n ? vals[e] : __int_as_float(0x7fc00000);
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t kk = score_key(v[j]);
      if (kk) {
        ++cnt;
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
  }
  uint32_t unused = 0;
  block_count_min_max<BLOCK>(cnt, kmin, kmax, unused, sm.red);
  const uint32_t n_valid = cnt;
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) o_idx[p] = -1;
    return;
  }

  uint32_t need = K;
  uint32_t lo = kmin, span = kmax - kmin;
  for (int round = 0; round < 4; ++round) {
    const int shift = max(0, bit_width(span) - 12);
    const int nb = (int)(span >> shift) + 1;
    for (int j = tid; j < nb; j += BLOCK) sm.hist[j] = 0u;
    __syncthreads();
    for (int e = tid; e < n; e += BLOCK) {
      const uint32_t kk = score_key(vals[e]);
      const uint32_t rel = kk - lo;
      if (kk && kk >= lo && rel <= span) atomicAdd(&sm.hist[rel >> shift], 1u);
    }
    __syncthreads();
    find_bin<BLOCK>(sm.hist, nb, need, sm.wsum, sm.sel);
    const uint32_t d = sm.sel[0];
    need -= sm.sel[1];
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
    const uint32_t kk = e < n ? score_key(vals[e]) : 0u;
    cgt += __popcll(__ballot(kk > T));
    ceq += __popcll(__ballot(kk == T));
  }
  if (lane == 0) {
    sm.wa[wave] = cgt;
    sm.wb[wave] = ceq;
  }
  __syncthreads();
  uint32_t eq_before = 0, sel_before = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t eqw = sm.wb[w];
    const uint32_t take = need > eq_before ? min(eqw, need - eq_before) : 0u;
    sel_before += sm.wa[w] + take;
    eq_before += eqw;
  }
  uint32_t run_eq = eq_before, run_sel = sel_before;
  for (int st = st0; st < st1; ++st) {
    const int e = st * 64 + lane;
    const uint32_t kk = e < n ? score_key(vals[e]) : 0u;
    const bool gt = kk > T;
    const bool eq = kk == T;
    const uint64_t beq = __ballot(eq);
    const bool sel = gt || (eq && run_eq + mbcnt(beq) < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t p = run_sel + mbcnt(bsel);
    if (sel && p < K) o_idx[p] = e;
    run_eq += __popcll(beq);
    run_sel += __popcll(bsel);
  }
  for (int p = (int)K + tid; p < top_k; p += BLOCK) o_idx[p] = -1;
}

template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void topk_rows_stream(const float* __restrict__ scores, int n_kv, int top_k,
                                                          int* __restrict__ out_idx) {
  __shared__ StreamSmem<BLOCK> sm;
  const long row = blockIdx.x;
  select_streaming<BLOCK>(sm, scores + row * n_kv, n_kv, top_k, out_idx + row * top_k);
}

// ---------------------------------------------------------------------------------------
// Register-resident select: thread t holds elements j * BLOCK + t (j < ITEMS) of the list,
// so a wave's lanes hold 64 consecutive elements for each j ("chunk" j * NW + wave, chunks in
// ascending element order). Finding T, the K-th largest key:
//  - K equal to the number of valid keys: T is their minimum;
//  - otherwise histogram rounds of 8192 bins over a shrinking key range [lo, lo + span]
//    (the first range is [min, max] of the valid keys); wave 0 finds the bin d holding the
//    need-th largest key. A round with shift 0 gives T = lo + d. When the bin's rank is its
//    largest or smallest key, one LDS max / min over the bin gives T; when the bin holds at
//    most 64 keys, wave 0 ranks them directly; else the next round narrows to the bin.
// The ordered compaction counts every chunk's keys > T and == T with ballots, wave 0 turns
// the counts (packed in one word) into output offsets, and each chunk is written with
// ballot + mbcnt. Keys == T are taken from the lowest index up until K are chosen. id_of(j)
// is the index written for item j.
// ---------------------------------------------------------------------------------------
template <int BLOCK, int ITEMS>
struct ResidentSmem {
  uint32_t hist[8192];
  uint32_t part[BLOCK];  // 16-byte aligned: follows hist
  uint4 red[BLOCK / 64 + 1];
  uint32_t cnt[ITEMS * (BLOCK / 64)];   // per chunk: (keys > T) << 16 | (keys == T)
  uint32_t eqb[ITEMS * (BLOCK / 64)];   // keys == T before the chunk
  uint32_t selb[ITEMS * (BLOCK / 64)];  // output slots before the chunk
  uint32_t list[64];
  uint32_t sel[3];
  uint32_t mm[2];   // max, min of one bin
  uint32_t nlist;
  uint32_t t_key;
  uint32_t eq_take;
};

// The K-th largest of the nonzero keys held in key[] (1 <= K <= n_valid, their count; kmin and
// kmax their extremes): radix rounds on the live range [lo, lo + span], at most 8192 LDS bins
// each, narrowed to the bin holding the K-th key. Uniform over the workgroup.
template <int BLOCK, int ITEMS>
__device__ __forceinline__ uint32_t resident_kth(ResidentSmem<BLOCK, ITEMS>& sm, const uint32_t (&key)[ITEMS],
                                                 uint32_t K, uint32_t n_valid, uint32_t kmin, uint32_t kmax) {
  constexpr int NB = 8192;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint4* h4 = reinterpret_cast<uint4*>(sm.hist);
  uint32_t T = kmin;  // every valid key is taken when K == n_valid
  if (K < n_valid) {
    uint32_t need = K;
    uint32_t lo = kmin, span = kmax - kmin;
    for (int round = 0; round < 4; ++round) {  // uniform over the workgroup
      const int shift = max(0, bit_width(span) - 13);
      for (int i = tid; i < NB / 4; i += BLOCK) h4[i] = make_uint4(0u, 0u, 0u, 0u);
      if (tid == 0) {
        sm.mm[0] = 0u;
        sm.mm[1] = 0xffffffffu;
        sm.nlist = 0u;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const uint32_t rel = key[j] - lo;
        if (key[j] && key[j] >= lo && rel <= span) atomicAdd(&sm.hist[rel >> shift], 1u);
      }
      __syncthreads();
      bin_parts<BLOCK, NB>(sm.hist, sm.part);
      __syncthreads();
      if (wave == 0) wave_find_in<NB>(sm.hist, wave_part_scan<BLOCK, NB>(sm.part), need, sm.sel);
      __syncthreads();
      const uint32_t d = sm.sel[0], cd = sm.sel[2];
      need -= sm.sel[1];
      lo += d << shift;
      if (shift == 0) {
        T = lo;
        break;
      }
      span = min(span - (d << shift), (1u << shift) - 1u);
      // T is the need-th largest of the cd keys in [lo, lo + span]
      if (need == 1 || need == cd) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
          const uint32_t rel = key[j] - lo;
          if (key[j] && key[j] >= lo && rel <= span) {
            if (need == 1) atomicMax(&sm.mm[0], key[j]);
            else atomicMin(&sm.mm[1], key[j]);
          }
        }
        __syncthreads();
        T = need == 1 ? sm.mm[0] : sm.mm[1];
        break;
      }
      if (cd <= 64) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
          const uint32_t rel = key[j] - lo;
          if (key[j] && key[j] >= lo && rel <= span) sm.list[atomicAdd(&sm.nlist, 1u)] = key[j];
        }
        __syncthreads();
        if (wave == 0) {
          const uint32_t mine = lane < (int)cd ? sm.list[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (int i = 0; i < (int)cd; ++i) {
            const uint32_t o = __builtin_amdgcn_readlane(mine, i);
            gt += o > mine;
            ge += o >= mine;
          }
          if (lane < (int)cd && gt < need && need <= ge) sm.t_key = mine;
        }
        __syncthreads();
        T = sm.t_key;
        break;
      }
    }
  }

  return T;
}

// Writes the K chosen keys' ids in item order (item j * BLOCK + tid of key[j]): every key > T
// and the first K - count(> T) keys == T, through ballot compaction, then -1 up to top_k.
template <int BLOCK, int ITEMS, typename IdOf>
__device__ __forceinline__ void resident_write(ResidentSmem<BLOCK, ITEMS>& sm, const uint32_t (&key)[ITEMS],
                                               uint32_t T, uint32_t K, int top_k, IdOf id_of,
                                               int* __restrict__ o_idx, float* __restrict__ o_val) {
  constexpr int NW = BLOCK / 64;
  constexpr int NCH = ITEMS * NW;  // chunks of 64
  constexpr int CPL = (NCH + 63) / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // per-chunk counts of keys > T and == T
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint32_t ngt = (uint32_t)__popcll(__ballot(key[j] > T));
    const uint32_t neq = (uint32_t)__popcll(__ballot(key[j] == T));
    if (lane == 0) sm.cnt[j * NW + wave] = (ngt << 16) | neq;
  }
  __syncthreads();
  if (wave == 0) {
    // lane l owns chunks [l * CPL, (l + 1) * CPL); counts stay below 2^16 in each half
    uint32_t v[CPL], local = 0;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane * CPL + k;
      v[k] = c < NCH ? sm.cnt[c] : 0u;
      local += v[k];
    }
    const uint32_t incl = wave_scan_up(local);
    const uint32_t total = lane_value(incl, 63);
    const uint32_t eq_take = K - (total >> 16);  // keys == T that are chosen
    uint32_t before = incl - local;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane * CPL + k;
      if (c < NCH) {
        const uint32_t eqb = before & 0xffffu;
        sm.eqb[c] = eqb;
        sm.selb[c] = (before >> 16) + min(eqb, eq_take);
      }
      before += v[k];
    }
    if (lane == 0) sm.eq_take = eq_take;
  }
  __syncthreads();
  const uint32_t eq_take = sm.eq_take;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int c = j * NW + wave;
    const uint32_t eqb = sm.eqb[c], selb = sm.selb[c];
    const bool gt = key[j] > T;
    const bool eq = key[j] == T;
    const bool sel = gt || (eq && eqb + mbcnt(__ballot(eq)) < eq_take);
    const uint64_t bsel = __ballot(sel);
    const uint32_t p = selb + mbcnt(bsel);
    if (sel && p < K) {
      o_idx[p] = id_of(j);
      if (o_val) o_val[p] = key_value(key[j]);
    }
  }
  for (int p = (int)K + tid; p < top_k; p += BLOCK) {
    o_idx[p] = -1;
    if (o_val) o_val[p] = -INFINITY;
  }
}

template <int BLOCK, int ITEMS, typename IdOf>
__device__ __forceinline__ void select_resident(ResidentSmem<BLOCK, ITEMS>& sm, const uint32_t (&key)[ITEMS],
                                                int top_k, IdOf id_of, int* __restrict__ o_idx,
                                                float* __restrict__ o_val) {
  const int tid = threadIdx.x;
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    if (key[j]) {
      ++cnt;
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  uint32_t unused = 0;
  block_count_min_max<BLOCK>(cnt, kmin, kmax, unused, sm.red);
  const uint32_t n_valid = cnt;
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) {
      o_idx[p] = -1;
      if (o_val) o_val[p] = -INFINITY;
    }
    return;
  }

  const uint32_t T = K < n_valid ? resident_kth<BLOCK, ITEMS>(sm, key, K, n_valid, kmin, kmax) : kmin;
  resident_write<BLOCK, ITEMS>(sm, key, T, K, top_k, id_of, o_idx, o_val);
}

// One workgroup per (segment, row) of the scores (stage 1 of the two-stage path, or the
// whole row), or per row of stage-1 candidates (CAND: values plus their indices).
template <int BLOCK, int ITEMS, bool CAND>
__global__ __launch_bounds__(BLOCK) void topk_rows_reg(const float* __restrict__ vals, long row_stride,
                                                       int seg_len, int n_total,
                                                       const int* __restrict__ cand, int top_k,
                                                       int* __restrict__ out_idx,
                                                       float* __restrict__ out_val) {
  __shared__ ResidentSmem<BLOCK, ITEMS> sm;
  const int tid = threadIdx.x;
  const int row = blockIdx.y, seg = blockIdx.x;
  const long base = (long)row * row_stride + (long)seg * seg_len;
  const int n = min(seg_len, n_total - seg * seg_len);
  const int idx_base = seg * seg_len;
  const long obase = ((long)row * gridDim.x + seg) * top_k;

  uint32_t key[ITEMS];
  int ci[CAND ? ITEMS : 1];
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
  if constexpr (CAND)
    select_resident<BLOCK, ITEMS>(sm, key, top_k, [&](int j) { return ci[j]; }, out_idx + obase,
                                  out_val ? out_val + obase : nullptr);
  else
    select_resident<BLOCK, ITEMS>(sm, key, top_k, [&](int j) { return idx_base + j * BLOCK + tid; },
                                  out_idx + obase, out_val ? out_val + obase : nullptr);
}

// ---------------------------------------------------------------------------------------
// Filtered path for few rows: many workgroups per row, then one per row.
//
// Stage 1 (topk_filter): workgroup (row, seg) takes a fixed sample of its row and picks a
// key G that at least `need` sampled valid keys reach: the lower edge of the histogram bin
// holding the need-th largest sampled key (G = 1, i.e. every valid key, when the sample holds
// no more than `need` valid keys). The sample is the whole row up to 2048 entries, else 512
// runs of 4 consecutive entries spread evenly over the row (runs keep the reads to at most
// 512 cache lines whatever the row length). `need` exceeds the sample's expected share of
// the top-k by several standard deviations, so the row usually holds at least top_k keys
// >= G. Every workgroup of a row computes the same G from the same sample. It then copies its
// segment's keys >= G with their indices, in index order, to the segment's slot of the
// workspace, and records how many it copied and how many of its keys are valid.
//
// Stage 2 (topk_filtered_select): the row's candidates, concatenated in segment order, are
// in ascending index order. If there are at least min(top_k, valid keys of the row) of them,
// the top-k of the row lies among them (every key of the top-k is >= the K-th largest key,
// which is >= G), so a register-resident select over the candidates gives the row's answer.
// Otherwise (the sample misjudged the row, or there are too many candidates to hold) the
// workgroup selects from the whole row with the streaming select. Both give the same
// unique result.
// ---------------------------------------------------------------------------------------
constexpr int kFilterBlock = 256, kFilterItems = 8, kFilterSeg = kFilterBlock * kFilterItems;
constexpr int kFilterSample = 2048, kFilterRun = 4;
constexpr int kSelectBlock = 1024, kSelectItems = 8, kFilterCap = kSelectBlock * kSelectItems;
constexpr int kFilterMaxSeg = kSelectBlock;
constexpr int kFilterMaxRows = 256;

template <int BLOCK, int ITEMS, int SAMPLE, int RUN>
__global__ __launch_bounds__(BLOCK) void topk_filter(const float* __restrict__ scores, int n_kv, int S, int rows,
                                                     uint32_t need, uint32_t* __restrict__ ckey,
                                                     int* __restrict__ cidx, uint32_t* __restrict__ ccnt) {
  constexpr int NW = BLOCK / 64, SEG = BLOCK * ITEMS, SPT = SAMPLE / BLOCK, NCH = ITEMS * NW;
  constexpr int NB = 4096, RUNS = SAMPLE / RUN;
  static_assert(NCH <= 64, "one lane per chunk in the offset scan");
  __shared__ uint32_t hist[NB];
  __shared__ uint4 s_red4[NW + 1];
  __shared__ uint32_t s_c[NCH];
  __shared__ __align__(16) uint32_t s_part[BLOCK];
  __shared__ uint32_t s_sel[3];
  __shared__ uint32_t s_tot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the S workgroups of a row share an XCD, whose L2 serves them the row's sample
  const int logical = xcd_remap(blockIdx.x, S * rows);
  const int row = logical / S, seg = logical - row * S;
  const float* rp = scores + (long)row * n_kv;
  const int e0 = seg * SEG;

  float v[ITEMS], sv[SPT];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int e = e0 + j * BLOCK + tid;
    v[j] = e < n_kv ? rp[e] : __int_as_float(0x7fc00000);
  }
  // sample entry i = j * BLOCK + tid: run i / RUN, offset i % RUN
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = j * BLOCK + tid;
    int pos;
    if (n_kv <= SAMPLE) pos = i;
    else pos = (int)(((long)(i / RUN) * (n_kv - RUN)) / (RUNS - 1)) + i % RUN;
    sv[j] = pos < n_kv ? rp[pos] : __int_as_float(0x7fc00000);
  }
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int i = tid; i < NB / 4; i += BLOCK) h4[i] = make_uint4(0u, 0u, 0u, 0u);

  // sample: count, min and max of the valid keys
  uint32_t sk[SPT];
  uint32_t cnt = 0, kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    sk[j] = score_key(sv[j]);
    if (sk[j]) {
      ++cnt;
      kmin = min(kmin, sk[j]);
      kmax = max(kmax, sk[j]);
    }
  }
  uint32_t unused = 0;
  block_count_min_max<BLOCK>(cnt, kmin, kmax, unused, s_red4);
  const uint32_t n_valid = cnt;
  uint32_t G = 1u;
  if (n_valid > need) {  // uniform over the workgroup
    const int shift = max(0, bit_width(kmax - kmin) - 12);
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (sk[j]) atomicAdd(&hist[(sk[j] - kmin) >> shift], 1u);
    __syncthreads();
    bin_parts<BLOCK, NB>(hist, s_part);
    __syncthreads();
    if (wave == 0) wave_find_in<NB>(hist, wave_part_scan<BLOCK, NB>(s_part), need, s_sel);
    __syncthreads();
    G = kmin + (s_sel[0] << shift);
  }

  // the segment's keys >= G, in index order; per chunk (candidates << 16) | valid keys
  uint32_t key[ITEMS];
  uint64_t bs[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    key[j] = score_key(v[j]);
    bs[j] = __ballot(key[j] >= G);
    const uint64_t bv = __ballot(key[j] != 0u);
    if (lane == 0) s_c[j * NW + wave] = ((uint32_t)__popcll(bs[j]) << 16) | (uint32_t)__popcll(bv);
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t mine = lane < NCH ? s_c[lane] : 0u;
    const uint32_t incl = wave_scan_up(mine);
    if (lane < NCH) s_c[lane] = (incl - mine) >> 16;
    if (lane == 63) s_tot = incl;
  }
  __syncthreads();
  const long slot = (long)row * S + seg;
  uint32_t* ok = ckey + slot * SEG;
  int* oi = cidx + slot * SEG;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    if (key[j] >= G) {
      const uint32_t p = s_c[j * NW + wave] + mbcnt(bs[j]);
      ok[p] = key[j];
      oi[p] = e0 + j * BLOCK + tid;
    }
  }
  if (tid == 0) {
    ccnt[slot * 2] = s_tot >> 16;
    ccnt[slot * 2 + 1] = s_tot & 0xffffu;
  }
}

template <int BLOCK, int ITEMS>
union FilterSelectSmem {
  ResidentSmem<BLOCK, ITEMS> res;
  StreamSmem<BLOCK> str;
};

template <int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void topk_filtered_select(const float* __restrict__ scores, int n_kv,
                                                              int top_k, int S, int seg_len, int cap_log,
                                                              const uint32_t* __restrict__ ckey,
                                                              const int* __restrict__ cidx,
                                                              const uint32_t* __restrict__ ccnt,
                                                              int* __restrict__ out_idx) {
  constexpr int SPL = BLOCK / 64;  // segments per lane in the count scan (S <= BLOCK)
  __shared__ FilterSelectSmem<BLOCK, ITEMS> sm;
  __shared__ uint32_t s_pre[BLOCK + 1];
  __shared__ uint32_t s_cnt[BLOCK];
  __shared__ uint32_t s_tv[3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the same row -> XCD grouping as the filter workgroups, so the candidates they wrote are
  // read from this XCD's L2
  const long row = xcd_remap(blockIdx.x, gridDim.x);
  int* o_idx = out_idx + row * top_k;
  const long row_base = row * S * (long)seg_len;

  // Optimistic read, issued before the counts arrive: item e reads slot e & (cap - 1) of
  // segment e >> cap_log (cap = 2^cap_log, S * cap <= BLOCK * ITEMS). It is the whole
  // candidate list when no segment copied more than cap keys.
  uint32_t key[ITEMS];
  int ci[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int e = j * BLOCK + tid;
    const int sg = e >> cap_log;
    const long a = sg < S ? row_base + (long)sg * seg_len + (e & ((1 << cap_log) - 1)) : row_base;
    key[j] = ckey[a];
    ci[j] = cidx[a];
  }
  if (wave == 0) {
    // lane l owns segments [l * SPL, (l + 1) * SPL)
    uint32_t c[SPL], local = 0, vloc = 0, cmax = 0;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sg = lane * SPL + k;
      c[k] = sg < S ? ccnt[(row * S + sg) * 2] : 0u;
      vloc += sg < S ? ccnt[(row * S + sg) * 2 + 1] : 0u;
      local += c[k];
      cmax = max(cmax, c[k]);
    }
    const uint32_t incl = wave_scan_up(local);
    uint32_t before = incl - local;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sg = lane * SPL + k;
      if (sg < S) {
        s_pre[sg] = before;
        s_cnt[sg] = c[k];
      }
      before += c[k];
    }
    const uint32_t vtot = wave_scan_up(vloc);
    cmax = lane_value(wave_scan(cmax, 0u, OpMax()), 63);
    if (lane == 63) {
      s_pre[S] = incl;
      s_tv[0] = incl;
      s_tv[1] = vtot;
      s_tv[2] = cmax;
    }
  }
  __syncthreads();
  const uint32_t T = s_tv[0], V = s_tv[1];
  const uint32_t K = min((uint32_t)top_k, V);
  if (T < K || T > (uint32_t)(BLOCK * ITEMS)) {  // uniform over the workgroup
    select_streaming<BLOCK>(sm.str, scores + row * n_kv, n_kv, top_k, o_idx);
    return;
  }
  if (s_tv[2] <= (1u << cap_log)) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = j * BLOCK + tid;
      const int sg = e >> cap_log;
      if (sg >= S || (uint32_t)(e & ((1 << cap_log) - 1)) >= s_cnt[min(sg, S - 1)]) key[j] = 0u;
    }
  } else {
    // a segment overflowed its slots: candidate e lives in the segment s with
    // s_pre[s] <= e < s_pre[s + 1]
    const int top_bit = 1 << (31 - __clz(S));
    long addr[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const uint32_t e = (uint32_t)(j * BLOCK + tid);
      int sg = 0;
      for (int b = top_bit; b > 0; b >>= 1)
        if (sg + b < S && s_pre[sg + b] <= e) sg += b;
      addr[j] = e < T ? row_base + (long)sg * seg_len + (e - s_pre[sg]) : row_base;
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      key[j] = ckey[addr[j]];
      ci[j] = cidx[addr[j]];
    }
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
      if ((uint32_t)(j * BLOCK + tid) >= T) key[j] = 0u;
  }
  select_resident<BLOCK, ITEMS>(sm.res, key, top_k, [&](int j) { return ci[j]; }, o_idx, nullptr);
}

// ---------------------------------------------------------------------------------------
// Selection over the candidates of the fused score -> top-k call: one workgroup per row.
//
// The score kernel left, for each wave w of the row (its range of G keys), e_w = min(v_w, m) of
// its valid keys in index order as (key, index) pairs (key 0 in the unused slots), its valid
// count v_w and, when it held more than m valid keys (truncated), a bound tau_w on every key it
// did not keep (the top of the 16-bit bin it was cut in). Let K = min(top_k, sum v_w) and T the K-th
// largest of the union U of the kept keys. A key a truncated wave did not keep is at most
// tau_w, so when tau_w < T it is below K keys of U and cannot be chosen: if every truncated
// wave has tau_w < T, the top-k of U is the top-k of the row. Otherwise the waves with
// tau_w >= T (all truncated waves when U holds fewer than K keys) are re-read whole from the
// stored scores and the selection runs again over that larger set; its K-th key is at least T,
// so every other truncated wave still lies below it and one re-read suffices. A set larger
// than the workgroup holds falls back to the streaming select over the stored row. Every
// route gives the row's unique answer. Candidates are concatenated in wave order, so in
// ascending index order, which the ordered output keeps.
// ---------------------------------------------------------------------------------------
template <int BLOCK, int ITEMS>
__global__ __launch_bounds__(BLOCK) void topk_cand_select(const float* __restrict__ scores, int n_kv, int top_k,
                                                          int n_w, int m, int G, const uint2* __restrict__ ckv,
                                                          const uint4* __restrict__ chdr, int* __restrict__ out_idx) {
  constexpr int NW = BLOCK / 64;
  constexpr int WPT = (kCandMaxWaves + BLOCK - 1) / BLOCK;  // waves (headers) per thread: tid * WPT + i
  __shared__ FilterSelectSmem<BLOCK, ITEMS> sm;
  __shared__ uint32_t s_pre[kCandMaxWaves + 1];
  __shared__ uint8_t s_off[kCandMaxWaves];    // wave re-read whole
  __shared__ uint4 s_red4[NW + 1];
  const int tid = threadIdx.x;
  const long row = blockIdx.x;
  int* o_idx = out_idx + row * top_k;
  const int slots = n_w * m;
  const long cbase = row * (long)slots;

  // candidates (issued first; a wave's slots past its kept count hold key 0) and headers
  uint32_t key[ITEMS];
  int ci[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int e = j * BLOCK + tid;
    const uint2 v = e < slots ? ckv[cbase + e] : make_uint2(0u, 0xffffffffu);
    key[j] = v.x;
    ci[j] = (int)v.y;
  }
  uint4 h[WPT];
  uint32_t vsum = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    h[i] = w < n_w ? chdr[row * n_w + w] : make_uint4(0u, 0u, 0u, 0u);
    vsum += h[i].y;
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
  block_count_min_max<BLOCK>(cnt, kmin, kmax, vsum, s_red4);
  const uint32_t n_u = cnt, n_valid = vsum;
  const uint32_t K = min((uint32_t)top_k, n_valid);
  if (K == 0) {
    for (int p = tid; p < top_k; p += BLOCK) o_idx[p] = -1;
    return;
  }
  uint32_t T = 0u;
  bool refine = n_u < K;  // uniform
  if (!refine) {
    T = K < n_u ? resident_kth<BLOCK, ITEMS>(sm.res, key, K, n_u, kmin, kmax) : kmin;
    bool mine = false;
#pragma unroll
    for (int i = 0; i < WPT; ++i) mine |= h[i].y > h[i].x && h[i].z >= T;  // truncated at or above T
    refine = __syncthreads_or(mine) != 0;
  }
  if (!refine) {
    resident_write<BLOCK, ITEMS>(sm.res, key, T, K, top_k, [&](int j) { return ci[j]; }, o_idx, nullptr);
    return;
  }
  // re-read the offending waves whole: wave w then contributes its whole key range
  uint32_t c[WPT], local = 0;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    const bool off = h[i].y > h[i].x && (n_u < K || h[i].z >= T);
    c[i] = w < n_w ? (off ? (uint32_t)min(G, n_kv - w * G) : h[i].x) : 0u;
    if (w < n_w) s_off[w] = off ? 1 : 0;
    local += c[i];
  }
  uint32_t total;
  uint32_t before = block_exclusive_scan<BLOCK>(local, sm.str.wsum, &total);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int w = tid * WPT + i;
    if (w < n_w) s_pre[w] = before;
    before += c[i];
  }
  if (tid == 0) s_pre[n_w] = total;
  __syncthreads();
  if (total > (uint32_t)(BLOCK * ITEMS)) {  // uniform
    select_streaming<BLOCK>(sm.str, scores + row * n_kv, n_kv, top_k, o_idx);
    return;
  }
  const int top_bit = 1 << (31 - __clz(n_w));
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const uint32_t e = (uint32_t)(j * BLOCK + tid);
    key[j] = 0u;
    ci[j] = -1;
    if (e < total) {
      int w = 0;
      for (int bb = top_bit; bb > 0; bb >>= 1)
        if (w + bb < n_w && s_pre[w + bb] <= e) w += bb;
      const int slot = (int)(e - s_pre[w]);
      if (s_off[w]) {
        const int t = w * G + slot;
        key[j] = score_key(scores[row * n_kv + t]);
        ci[j] = t;
      } else {
        const uint2 v = ckv[cbase + (long)w * m + slot];
        key[j] = v.x;
        ci[j] = (int)v.y;
      }
    }
  }
  __syncthreads();
  select_resident<BLOCK, ITEMS>(sm.res, key, top_k, [&](int j) { return ci[j]; }, o_idx, nullptr);
}

std::atomic<int> g_topk_cand_block{0};

hipError_t launch_topk_cand(const float* scores, int* idx, int rows, int n_kv, int top_k,
                            const ScoreTopkPlan& plan, const CandOut& cand, hipStream_t stream) {
  const int tuned = g_topk_cand_block.load(std::memory_order_relaxed);
  const int G = 64 * plan.iters;
#define DSA_CAND_SELECT(BL, IT)                                                                      \
  static_assert(BL * IT >= kCandCap, "one select workgroup holds the candidate union");             \
  hipLaunchKernelGGL((topk_cand_select<BL, IT>), dim3(rows), dim3(BL), 0, stream, scores, n_kv, top_k, \
                     plan.n_w, plan.m, G, cand.kv, cand.hdr, idx)
  if (plan.wide) {
    static_assert(1024 * 16 == kCandCapWide, "the wide select holds kCandCapWide candidates");
    DSA_CAND_SELECT(1024, 16);
  } else if (tuned == 256) {
    DSA_CAND_SELECT(256, 32);
  } else if (tuned == 512) {
    DSA_CAND_SELECT(512, 16);
  } else {
    DSA_CAND_SELECT(1024, 8);
  }
#undef DSA_CAND_SELECT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static constexpr int kResidentMax = 32768;  // longest segment held in registers by one workgroup
static constexpr int kCandMax = 32768;      // candidates of one row in the second stage
static constexpr int kSegTarget = 8192;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Sampled keys that G must cover: the sample's expected share of the top-k, mu, plus four
// standard deviations (at most sqrt(mu) for a sample drawn without replacement) and 8.
static uint32_t filter_need(int n_kv, int top_k) {
  const int m = n_kv < kFilterSample ? n_kv : kFilterSample;
  const double mu = (double)top_k * m / n_kv;
  return (uint32_t)ceil(mu + 4.0 * sqrt(mu)) + 8u;
}

TopkPlan plan_topk(int rows, int n_kv, int top_k, int path) {
  TopkPlan p{0, 1, n_kv, 0u, 0};
  size_t ws = 0;
  // two-stage: segments of about kSegTarget entries, each keeping top_k candidates, but no
  // more candidates per row than one register-resident stage-2 pass holds
  int S2 = (n_kv + kSegTarget - 1) / kSegTarget;
  if (S2 > kCandMax / top_k) S2 = kCandMax / top_k;
  if (S2 < 2) S2 = 2;
  int seg2 = (n_kv + S2 - 1) / S2;
  seg2 = (seg2 + 63) / 64 * 64;
  S2 = (n_kv + seg2 - 1) / seg2;
  const bool two_ok = S2 >= 2 && (long)S2 * top_k <= kCandMax && seg2 <= kResidentMax && seg2 >= 2 * top_k;
  if (two_ok) {
    const size_t cand = (size_t)rows * S2 * top_k;
    ws = std::max(ws, align256(cand * sizeof(int)) + align256(cand * sizeof(float)));
  }
  // filtered: segments of kFilterSeg entries; expected candidates (about top_k plus the
  // margin) must fit one register-resident select
  const int Sf = (n_kv + kFilterSeg - 1) / kFilterSeg;
  const bool filt_ok = rows <= kFilterMaxRows && Sf <= kFilterMaxSeg && 2L * top_k <= kFilterCap;
  if (filt_ok) {
    const size_t slots = (size_t)rows * Sf * kFilterSeg;
    ws = std::max(ws, 2 * align256(slots * 4) + align256((size_t)rows * Sf * 2 * 4));
  }
  p.ws_bytes = ws;

  int kind = 0;
  if (path == 2 && two_ok) kind = 1;
  else if (path == 3 && filt_ok) kind = 2;
  else if (path == 0) {
    // few rows leave most CUs idle with one workgroup per row
    if (filt_ok && rows <= 64 && n_kv >= 16384) kind = 2;
    else if (two_ok && n_kv > kResidentMax) kind = 1;
  }
  p.kind = kind;
  if (kind == 1) {
    p.segments = S2;
    p.seg_len = seg2;
  } else if (kind == 2) {
    p.segments = Sf;
    p.seg_len = kFilterSeg;
    p.need = filter_need(n_kv, top_k);
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
  else DSA_TOPK_REG(1024, 32);
#undef DSA_TOPK_REG
}

// ---------------------------------------------------------------------------------------
// Scratch for callers that cannot allocate (dsa_topk_noalloc): a file-scope device array,
// one copy per GPU, held from the library's load until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is looked up with hipGetSymbolAddress once per device, with that device
// current, and kept. Every path writes what it later reads (candidate keys and indices,
// per-segment counts, stage-1 results), so nothing needs clearing between calls; calls that
// overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t topk_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_dev[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_topk(const float* scores, int* idx, int rows, int n_kv, int top_k,
                       const TopkPlan& plan, void* workspace, hipStream_t stream) {
  if (plan.kind == 0) {
    if (n_kv <= kResidentMax)
      launch_rows_t<false>(scores, n_kv, n_kv, n_kv, 1, rows, nullptr, top_k, idx, nullptr, stream);
    else
      hipLaunchKernelGGL((topk_rows_stream<1024>), dim3(rows), dim3(1024), 0, stream, scores, n_kv, top_k, idx);
    return hipGetLastError();
  }
  if (plan.kind == 2) {
    const int S = plan.segments;
    const size_t slots = (size_t)rows * S * kFilterSeg;
    char* w = reinterpret_cast<char*>(workspace);
    uint32_t* ckey = reinterpret_cast<uint32_t*>(w);
    int* cidx = reinterpret_cast<int*>(w + align256(slots * 4));
    uint32_t* ccnt = reinterpret_cast<uint32_t*>(w + 2 * align256(slots * 4));
    hipLaunchKernelGGL((topk_filter<kFilterBlock, kFilterItems, kFilterSample, kFilterRun>), dim3(S * rows),
                       dim3(kFilterBlock), 0, stream, scores, n_kv, S, rows, plan.need, ckey, cidx, ccnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int cap_log = 0;  // slots per segment read before the counts are known
    while ((2 << cap_log) <= kFilterSeg && (long)S * (2 << cap_log) <= kFilterCap) ++cap_log;
    hipLaunchKernelGGL((topk_filtered_select<kSelectBlock, kSelectItems>), dim3(rows), dim3(kSelectBlock), 0,
                       stream, scores, n_kv, top_k, S, kFilterSeg, cap_log, ckey, cidx, ccnt, idx);
    return hipGetLastError();
  }
  const size_t cand = (size_t)rows * plan.segments * top_k;
  int* ws_idx = reinterpret_cast<int*>(workspace);
  float* ws_val = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(cand * sizeof(int)));
  launch_rows_t<false>(scores, n_kv, plan.seg_len, n_kv, plan.segments, rows, nullptr, top_k, ws_idx, ws_val,
                       stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int m = plan.segments * top_k;
  launch_rows_t<true>(ws_val, m, m, m, 1, rows, ws_idx, top_k, idx, nullptr, stream);
  return hipGetLastError();
}

}  // namespace dsa
