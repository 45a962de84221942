// Lightning-indexer scores (ik_llama_opt commit log, sub-commits "Add GLM-5.2/DeepSeek-V3.2
// DSA lightning indexer" and "decode-correct via persistent indexer-K cache"):
//   S[b,i,t] = scale * sum_h w[b,i,h] * relu(sum_d q[b,i,h,d] * k[b,t,d]),  -inf if masked.
//
// Three kernels:
//   index_score_plain        any dtype / shape, 16 lanes per key (fp32 inputs, odd shapes)
//   index_score_decode_mfma  16-bit inputs, D = 128, H <= 32, few queries per sequence:
//                            each wave owns 64 keys per step, the 32 heads sit on the MFMA M
//                            dimension, relu + head weights + head sum run in the epilogue.
//   index_score_prefill_mfma 16-bit inputs, D = 128, H <= 32, many queries: a 64-key tile is
//                            staged in LDS once and shared by 8 queries (2 per wave).
// Keys are read from HBM exactly once per (query block, key) with coalesced 16-byte loads and
// re-laid out through XOR-swizzled LDS into the MFMA operand layout.
#include "common.h"
#include "kernels.h"

#include <limits.h>
#include <math.h>

namespace dsa {

std::atomic<int> g_score_cpw{0};            // 64-key chunks per wave of the decode kernel (0 automatic)
std::atomic<int> g_score_prefill_waves{0};  // waves per block of the prefill kernel (0 automatic)
constexpr int kPrefillWaves = 8;

// Attention-sink range [lo, hi) of sequence b (ik_llama_opt log, "per-sequence attention sink"
// and "UPDATE 6" sub-commits: the first n_sink keys of the query's own sequence, counted from
// its first present position, get a large additive boost so that top-k always keeps them).
struct SinkRange {
  int lo, hi;
  float boost;
  __device__ __forceinline__ float add(int t, float v) const { return t >= lo && t < hi ? v + boost : v; }
};
__device__ __forceinline__ SinkRange sink_range(const ScoreArgs& s, int b) {
  SinkRange r{0, 0, s.boost};
  if (s.n > 0) {
    r.lo = s.start ? s.start[b] : 0;
    r.hi = (int)min((long)r.lo + s.n, (long)INT_MAX);
  }
  return r;
}

// Keys [0, limit) of query i of sequence b (row bi) are scored, the rest are -inf: keys after
// the query's position or past the cache's length (ik_llama_opt log, lightning-indexer
// sub-commit: causal mask). With pools of kpool tokens (vllm-rdna "Glm5Next" PR, kpool
// indexer) key p holds tokens kpool p .. kpool p + kpool - 1; it is in the cache when all of
// them are and visible once its last one is: limit = min(floor(len / kpool),
// floor((pos + 1) / kpool)), with len and pos in tokens.
__device__ __forceinline__ long floor_div(long a, long m) { return a >= 0 ? a / m : -((-a + m - 1) / m); }
__device__ __forceinline__ int key_limit(const int* kv_len, const int* q_pos, long bi, int b, int i, int n_q,
                                         int n_kv, int kpool) {
  const long cap = (long)n_kv * kpool;
  const long len = kv_len ? min((long)kv_len[b], cap) : cap;
  const long pos = q_pos ? (long)q_pos[bi] : len - n_q + i;
  const long lim = min(floor_div(len, kpool), floor_div(pos + 1, kpool));
  return (int)max(0L, min(lim, (long)n_kv));
}

// ---------------------------------------------------------------------------------------
// plain kernel: grid (ceil(n_kv / 64), B * n_q), 256 threads. A 16-lane group scores one key at
// a time, four keys per group: lane l takes dims l, l + 16, ... of the key's row, so each load
// of a group reads consecutive values, and every head's dot product is summed with xor shuffles
// inside the group.
// ---------------------------------------------------------------------------------------
constexpr int kPlainKeys = 64;

template <typename T>
__global__ __launch_bounds__(256) void index_score_plain(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ w,
    const int* __restrict__ kv_len, const int* __restrict__ q_pos, float* __restrict__ scores,
    int n_q, int H, int D, int n_kv, float scale, ScoreArgs sink) {
  extern __shared__ float qs[];  // [H][D] of this query
  const int bi = blockIdx.y;
  const int b = bi / n_q, i = bi - b * n_q;
  const T* qp = q + (long)bi * H * D;
  for (int e = threadIdx.x; e < H * D; e += blockDim.x) qs[e] = load_as_f32(qp, e);
  __syncthreads();
  const int limit = key_limit(kv_len, q_pos, bi, b, i, n_q, n_kv, sink.kpool);
  float* out = scores + (long)bi * n_kv;
  const float* wp = w + (long)bi * H;
  const SinkRange sk = sink_range(sink, b);
  const int grp = threadIdx.x >> 4, l = threadIdx.x & 15;
  for (int kk = 0; kk < kPlainKeys / 16; ++kk) {
    const int t = blockIdx.x * kPlainKeys + 16 * kk + grp;  // the same in the group's 16 lanes
    if (t >= n_kv) break;
    if (t >= limit) {
      if (l == 0) out[t] = -INFINITY;
      continue;
    }
    const T* kp = k + ((long)b * n_kv + t) * D;
    float s = 0.f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.f;
      for (int d = l; d < D; d += 16) dot = fmaf(qs[h * D + d], load_as_f32(kp, d), dot);
      dot += shfl_xor(dot, 8);
      dot += shfl_xor(dot, 4);
      dot += shfl_xor(dot, 2);
      dot += shfl_xor(dot, 1);
      s = fmaf(wp[h], fmaxf(dot, 0.f), s);
    }
    if (l == 0) out[t] = sk.add(t, scale * s);
  }
}

// ---------------------------------------------------------------------------------------
// MFMA helpers. v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[l%16][8*(l/16)+j] and
// B[8*(l/16)+j][l%16] (j = 0..7) and receives D[4*(l/16)+e][l%16] (e = 0..3).
// ---------------------------------------------------------------------------------------
template <typename T16> struct Mma16;
template <> struct Mma16<bf16_t> {
  static __device__ __forceinline__ f32x4 run(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma16<f16_t> {
  static __device__ __forceinline__ f32x4 run(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// One 128-dim key row is 256 bytes = 16 chunks of 16 bytes. In LDS, chunk c of tile row r
// sits at position c ^ (r & 15): the 16 lanes that read the same chunk of 16 consecutive
// rows then hit 16 different 16-byte bank groups.
__device__ __forceinline__ int key_lds_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// Query operand of one wave: heads 16*mt + (lane%16), k-step s covers dims 32*s + 8*(lane/16) .. +8.
// Heads past H load head H-1, so that the loads stay unconditional.
template <typename T16>
__device__ __forceinline__ void load_q_operand(const T16* q_bi, int H, int lane, i32x4 (&qa)[2][4]) {
  const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int head = min(16 * mt + r16, H - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qa[mt][s] = *reinterpret_cast<const i32x4*>(reinterpret_cast<const uint8_t*>(q_bi) +
                                                  head * 256 + (4 * s + g) * 16);
  }
}

// Weights of the accumulator rows a lane holds: heads 16*mt + 4*(lane/16) + e (clamped to
// H-1 like the query).
__device__ __forceinline__ void load_w_rows(const float* w_bi, int H, int lane, float (&wr)[2][4]) {
  const int g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) wr[mt][e] = w_bi[min(16 * mt + 4 * g + e, H - 1)];
}

// relu on the bit pattern: a set sign bit (negative values, -0.0, negative NaNs) gives +0.0,
// everything else passes unchanged. One integer max, where fmaxf would first quiet both
// operands.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// relu, head weight and the in-lane part of the head sum of one 16-key N tile: the lane's
// 8 accumulator rows (heads 4*(lane/16) + e and 16 + 4*(lane/16) + e) of key column lane%16.
// With fewer than 32 heads, rows past H (which hold copies of head H-1) are left out.
template <bool FULLH>
__device__ __forceinline__ float head_partial(const f32x4& a0, const f32x4& a1, const float (&wr)[2][4],
                                             int H, int g) {
  float p = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (FULLH) {
      p = fmaf(wr[0][e], relu(a0[e]), p);
      p = fmaf(wr[1][e], relu(a1[e]), p);
    } else {
      p += 4 * g + e < H ? wr[0][e] * relu(a0[e]) : 0.f;
      p += 16 + 4 * g + e < H ? wr[1][e] * relu(a1[e]) : 0.f;
    }
  }
  return p;
}

// Finishes the head sums of four N tiles at once: p[nt] holds lane row g = lane/16's part of
// tile nt. Afterwards lane (g, c) holds the full sum of tile g at column c. Two exchanges
// between the wave halves give the lower half tiles 0 and 1 and the upper half tiles 2 and
// 3 summed over both halves; one exchange between neighbouring 16-lane rows finishes them.
__device__ __forceinline__ uint32_t fbits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float tile_reduce(float p0, float p1, float p2, float p3) {
  // v_permlane32_swap: lanes 32..63 of the first operand trade places with lanes 0..31 of
  // the second, so x[0] + x[1] sums lane i with lane i ^ 32 of the pair (p0 | p2).
  const auto x = __builtin_amdgcn_permlane32_swap(fbits(p0), fbits(p2), false, false);
  const auto y = __builtin_amdgcn_permlane32_swap(fbits(p1), fbits(p3), false, false);
  const float a = __uint_as_float(x[0]) + __uint_as_float(x[1]);  // rows 0,1: tile 0; rows 2,3: tile 2
  const float c = __uint_as_float(y[0]) + __uint_as_float(y[1]);  // rows 0,1: tile 1; rows 2,3: tile 3
  // v_permlane16_swap: odd 16-lane rows of the first operand trade places with even rows
  // of the second.
  const auto z = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(c), false, false);
  return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// ---------------------------------------------------------------------------------------
// decode: grid (key blocks, B * n_q), 4 waves; wave w of block x handles the 64-key chunks
// ((x * ITERS + it) * 4 + w) for it < ITERS. Each wave keeps two chunks of loads in flight in
// ping-pong registers. The code between the loads and their use has no branches: the chunk
// loop is fully unrolled (ITERS is a template argument) and every load is unconditional,
// because at a join of paths with different loads in flight the compiler's wait counting
// falls back to waiting for all of them, the next chunk's included. Rows past the scored
// range are clamped to the last scored row (row 0 when nothing is scored), so every load
// reads real data and chunks past the range cost no extra HBM traffic; their scores are
// replaced by -inf at the store. A wave only reads the LDS tile it wrote itself, so waves
// never wait for each other: LDS operations of one wave execute in issue order, and a
// compiler-only fence keeps that order in the code. The key loads are nontemporal (the nt
// cache policy): every key row is read once per call, and streaming them past the caches'
// normal replacement measured 50.8 -> 46.2 us on 32 x 32768 keys (a plain read of 1 GiB
// reaches about 6.9 TB/s this way against 6.1 TB/s with default loads).
// ---------------------------------------------------------------------------------------
constexpr int kDecWaves = 4;

__device__ __forceinline__ void wave_lds_order() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

//
// With CAND (the fused score -> top-k call) each wave walks ITERS consecutive chunks, so that
// its keys form one range: range w * gridDim.x + x for wave w of block x, so that blocks
// running side by side read neighbouring ranges (ranges 4x .. 4x + 3 of block x measured 57.5
// against 56.4 us for the fused call on 32 x 32768 keys). After its stores the wave writes m
// of its range's keys as candidates for the selection: every key whose upper 16 bits exceed
// those of the m-th largest key, then keys sharing those 16 bits in index order (the keys of
// the stored scores, so the selection over the candidates and over the stored row agree bit
// for bit). The header's bound on the keys left out is then the top of that 16-bit bin;
// deciding 16 bits instead of all 32 halves the ballot rounds (fused call 58.0 -> 57.2 us).
template <typename T16, int ITERS, bool FULLH, bool CAND>
__global__ __launch_bounds__(256, 2) void index_score_decode_mfma(
    const T16* __restrict__ q, const T16* __restrict__ k, const float* __restrict__ w,
    const int* __restrict__ kv_len, const int* __restrict__ q_pos, float* __restrict__ scores,
    int n_q, int H, int n_kv, float scale, ScoreArgs sink, CandOut cand) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDecWaves][64 * 256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int bi = blockIdx.y;
  const int b = bi / n_q, i = bi - b * n_q;
  const int limit = key_limit(kv_len, q_pos, bi, b, i, n_q, n_kv, sink.kpool);  // keys [0, limit) are scored
  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(k) + (long)b * n_kv * 256;
  float* out = scores + (long)bi * n_kv;
  uint8_t* my = lds[wave];

  // chunk it of this wave starts at key kb(it)
  auto kb_of = [&](int it) {
    return CAND ? ((int)(wave * gridDim.x + blockIdx.x) * ITERS + it) * 64
                : ((int)(blockIdx.x * ITERS + it) * kDecWaves + wave) * 64;
  };
  const int last = max(limit - 1, 0);
  auto fetch = [&](int kb, i32x4(&pre)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = min(kb + 4 * j + g, last);
      pre[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kseq + (long)row * 256 + r16 * 16));
    }
  };

  // query and weights first: loads complete in issue order, so the first chunk's MFMAs
  // wait for that chunk only
  i32x4 qa[2][4];
  float wr[2][4];
  i32x4 pre[2][16];
  load_q_operand(q + (long)bi * H * 128, H, lane, qa);
  load_w_rows(w + (long)bi * H, H, lane, wr);
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order: query, weights, chunk 0, chunk 1
  fetch(kb_of(0), pre[0]);
  __builtin_amdgcn_sched_barrier(0);
  if (ITERS > 1) fetch(kb_of(1), pre[1]);
  __builtin_amdgcn_sched_barrier(0);

  // chunks past n_kv (in the last block) compute on clamped rows and store nothing
  float res[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    i32x4(&p)[16] = pre[it & 1];
    wave_lds_order();  // the previous chunk's tile reads stay before these writes
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 4 * j + g;
      *reinterpret_cast<i32x4*>(my + key_lds_off(r, r16)) = p[j];
    }
    if (it + 2 < ITERS) fetch(kb_of(it + 2), p);  // two chunks ahead, into the freed registers
    __builtin_amdgcn_sched_barrier(0);
    wave_lds_order();
    float sc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const i32x4 kv = *reinterpret_cast<const i32x4*>(my + key_lds_off(nt * 16 + r16, 4 * s + g));
        a0 = Mma16<T16>::run(qa[0][s], kv, a0);
        a1 = Mma16<T16>::run(qa[1][s], kv, a1);
      }
      sc[nt] = head_partial<FULLH>(a0, a1, wr, H, g);
    }
    res[it] = tile_reduce(sc[0], sc[1], sc[2], sc[3]);  // lane l: key kb + l
  }
  // stores last: a store guard is a branch, and the code-sinking pass would move the loads
  // of a later chunk past it, next to their use
  const SinkRange sk = sink_range(sink, b);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int t = kb_of(it) + lane;
    if (t < n_kv) out[t] = t < limit ? sk.add(t, scale * res[it]) : -INFINITY;
  }
  if constexpr (CAND) {
    // keys of the stored scores (0: masked or past the row)
    uint32_t key[ITERS];
    uint32_t nv = 0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int t = kb_of(it) + lane;
      key[it] = (t < n_kv && t < limit) ? score_key(sk.add(t, scale * res[it])) : 0u;
      nv += (uint32_t)__popcll(__ballot(key[it] != 0u));
    }
    // the 16-bit prefix p of the m-th largest key, by deciding its bits from the top: the
    // largest prefix with at least m keys at or above it. Keys with a larger prefix (fewer than
    // m) are kept, then keys of prefix p in index order up to m; every key left out is at most
    // z = p << 16 | 0xffff, the bound the header carries (with nv <= m every valid key is kept)
    const uint32_t m = (uint32_t)cand.m;
    uint32_t pb = 0u, take_eq = 0xffffffffu;
    if (nv > m) {
      for (int bit = 15; bit >= 0; --bit) {
        const uint32_t c = pb | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) cnt += (uint32_t)__popcll(__ballot((key[it] >> 16) >= c));
        if (cnt >= m) pb = c;
      }
      uint32_t nab = 0;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) nab += (uint32_t)__popcll(__ballot((key[it] >> 16) > pb));
      take_eq = m - nab;  // keys of prefix pb that are kept, the lowest indices first
    }
    const int nw = (int)gridDim.x * kDecWaves;
    const long slot = (long)bi * nw + (long)wave * gridDim.x + blockIdx.x;
    uint2* okv = cand.kv + slot * m;  // (key, index) in one 8-byte store
    uint32_t eq_before = 0, sel_before = 0;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const bool inb = key[it] != 0u && (key[it] >> 16) == pb;
      const uint64_t eqm = __ballot(inb);
      const bool sel = (key[it] >> 16) > pb || (inb && eq_before + mbcnt(eqm) < take_eq);
      const uint64_t selm = __ballot(sel);
      if (sel) {
        const uint32_t p = sel_before + mbcnt(selm);
        okv[p] = make_uint2(key[it], (uint32_t)(kb_of(it) + lane));
      }
      eq_before += (uint32_t)__popcll(eqm);
      sel_before += (uint32_t)__popcll(selm);
    }
    // slots past the kept keys hold key 0 (invalid), so the selection reads the candidates
    // without waiting for the headers
    for (uint32_t p = sel_before + lane; p < m; p += 64) okv[p] = make_uint2(0u, 0u);
    if (lane == 0) cand.hdr[slot] = make_uint4(min(nv, m), nv, nv > m ? (pb << 16 | 0xffffu) : 0u, 0u);
  }
}

// ---------------------------------------------------------------------------------------
// prefill: grid (query blocks, key spans, B), NWV waves x 2 queries. Every block walks its key
// span in 64-key tiles held in two LDS buffers; the next tile is fetched into registers while
// the current one feeds the MFMAs.
// ---------------------------------------------------------------------------------------
constexpr int kPreQPW = 2;  // queries per wave

template <typename T16, int NWV, bool FULLH>
__global__ __launch_bounds__(NWV * 64) void index_score_prefill_mfma(
    const T16* __restrict__ q, const T16* __restrict__ k, const float* __restrict__ w,
    const int* __restrict__ kv_len, const int* __restrict__ q_pos, float* __restrict__ scores,
    int n_q, int H, int n_kv, int key_span, float scale, ScoreArgs sink) {
  constexpr int kPreQB = NWV * kPreQPW;     // queries per block
  constexpr int kCPT = 1024 / (NWV * 64);  // 16-byte tile chunks each thread stages
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][64 * 256];
  __shared__ int s_limit[kPreQB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int b = blockIdx.z;
  // query blocks in descending order: workgroups are dispatched x fastest, and with queries at
  // increasing positions (a causal prefill chunk) the later query blocks hold more keys of the
  // diagonal key spans, so the heaviest workgroups of a span start first and the lightest (down
  // to spans wholly past every query of the block) fill the last gaps
  const int q0 = (gridDim.x - 1 - blockIdx.x) * kPreQB;
  if (tid < kPreQB) {
    const int qi = q0 + tid;
    s_limit[tid] = qi < n_q ? key_limit(kv_len, q_pos, (long)b * n_q + qi, b, qi, n_q, n_kv, sink.kpool) : 0;
  }
  __syncthreads();
  int kmax = 0;
#pragma unroll
  for (int j = 0; j < kPreQB; ++j) kmax = max(kmax, s_limit[j]);

  const int kbeg = blockIdx.y * key_span;
  const SinkRange sk = sink_range(sink, b);
  const int kend = min(n_kv, kbeg + key_span);
  const int kc_end = min(kend, kmax);  // keys [kbeg, kc_end) need the contraction

  // queries of this wave
  int qi[kPreQPW], lim[kPreQPW];
  i32x4 qa[kPreQPW][2][4];
  float wr[kPreQPW][2][4];
#pragma unroll
  for (int qq = 0; qq < kPreQPW; ++qq) {
    qi[qq] = q0 + wave * kPreQPW + qq;
    lim[qq] = s_limit[wave * kPreQPW + qq];
    if (qi[qq] < n_q) {
      const long bi = (long)b * n_q + qi[qq];
      load_q_operand(q + bi * H * 128, H, lane, qa[qq]);
      load_w_rows(w + bi * H, H, lane, wr[qq]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) qa[qq][mt][s] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) wr[qq][mt][e] = 0.f;
    }
  }

  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(k) + (long)b * n_kv * 256;
  // tile staging: thread tid copies chunks (j * NWV * 64 + tid), j < kCPT, of the 64 x 16
  // chunk tile
  i32x4 pre[kCPT];
  auto issue = [&](int kb) {
#pragma unroll
    for (int j = 0; j < kCPT; ++j) {
      const int r = j * (NWV * 4) + (tid >> 4);
      const int row = kb + r;
      pre[j] = row < kc_end ? *reinterpret_cast<const i32x4*>(kseq + (long)row * 256 + (tid & 15) * 16)
                            : i32x4{0, 0, 0, 0};
    }
  };
  const int ntiles = kc_end > kbeg ? (kc_end - kbeg + 63) / 64 : 0;
  if (ntiles > 0) issue(kbeg);
  // Software pipeline over the four 16-key N tiles of a key tile: the 16 MFMAs of N tile nt are
  // issued one by one, each followed by two VALU operations (relu, weighted add) of N tile
  // nt - 1's epilogue, so the matrix pipe and the vector ALU work at the same time within the
  // wave; the operands of N tile nt + 1 are read from LDS while N tile nt computes. The last N
  // tile's epilogue, the head-sum reduction and the stores of a key tile run during the next key
  // tile's first 16 MFMAs, so that between two barriers no epilogue is left without products to
  // hide behind. sched_barrier pins this order.
  static_assert(kPreQPW == 2, "the pipeline pairs 16 MFMAs with 16 epilogue steps");
  float sc[kPreQPW][4];
  i32x4 kv[2][4];
  f32x4 acc[2][kPreQPW][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int qq = 0; qq < kPreQPW; ++qq)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[a][qq][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto read_tile = [&](const uint8_t* buf, int nt, i32x4(&dst)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      dst[s] = *reinterpret_cast<const i32x4*>(buf + key_lds_off(nt * 16 + r16, 4 * s + g));
  };
  // MFMA i of an N tile: k-step i / 4, query (i / 2) % 2, head tile i % 2
  auto mma_step = [&](int i, const i32x4(&op)[4], f32x4(&a)[kPreQPW][2]) {
    const int s = i >> 2, qq = (i >> 1) & 1, mt = i & 1;
    a[qq][mt] = Mma16<T16>::run(qa[qq][mt][s], op[s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : a[qq][mt]);
  };
  // epilogue step i of an N tile: query i / 8, head tile i % 2, accumulator row (i / 2) % 4
  auto epi_step = [&](int i, const f32x4(&a)[kPreQPW][2], float(&p)[kPreQPW]) {
    const int qq = i >> 3, mt = i & 1, e = (i >> 1) & 3;
    const float v = relu(a[qq][mt][e]);
    if (FULLH) p[qq] = fmaf(wr[qq][mt][e], v, p[qq]);
    else p[qq] += 16 * mt + 4 * g + e < H ? wr[qq][mt][e] * v : 0.f;
  };
  // the finished key tile at kb_done: head sums across lanes, then the stores
  auto finish = [&](int kb_done) {
    const int t = kb_done + lane;
#pragma unroll
    for (int qq = 0; qq < kPreQPW; ++qq) {
      // cross-lane, so outside the store guard: every lane takes part
      const float v = tile_reduce(sc[qq][0], sc[qq][1], sc[qq][2], sc[qq][3]);
      if (qi[qq] < n_q && t < kend)
        scores[((long)b * n_q + qi[qq]) * n_kv + t] = t < lim[qq] ? sk.add(t, scale * v) : -INFINITY;
    }
  };
  for (int tile = 0; tile < ntiles; ++tile) {
    const int kb = kbeg + tile * 64;
    uint8_t* buf = lds[tile & 1];
#pragma unroll
    for (int j = 0; j < kCPT; ++j) {
      const int r = j * (NWV * 4) + (tid >> 4);
      *reinterpret_cast<i32x4*>(buf + key_lds_off(r, tid & 15)) = pre[j];
    }
    __syncthreads();
    if (tile + 1 < ntiles) issue(kb + 64);
    read_tile(buf, 0, kv[0]);
    read_tile(buf, 1, kv[1]);
    {
      // N tile 0, with the previous key tile's last epilogue (on the first key tile it works on
      // the zeroed accumulators and its result is never stored)
      float p[kPreQPW] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        mma_step(i, kv[0], acc[0]);
        epi_step(i, acc[1], p);
      }
      sc[0][3] = p[0];
      sc[1][3] = p[1];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tile > 0) finish(kb - 64);
#pragma unroll
    for (int nt = 1; nt < 4; ++nt) {
      __builtin_amdgcn_sched_barrier(0);
      if (nt + 1 < 4) read_tile(buf, nt + 1, kv[(nt + 1) & 1]);  // N tile nt - 1's operands are consumed
      float p[kPreQPW] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        mma_step(i, kv[nt & 1], acc[nt & 1]);
        epi_step(i, acc[(nt - 1) & 1], p);
      }
      sc[0][nt - 1] = p[0];
      sc[1][nt - 1] = p[1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (ntiles > 0) {  // the last key tile's last epilogue and its stores
    float p[kPreQPW] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) epi_step(i, acc[1], p);
    sc[0][3] = p[0];
    sc[1][3] = p[1];
    finish(kbeg + (ntiles - 1) * 64);
  }
  // keys of the span past every query's limit are masked for all of them
  const int mstart = max(kbeg, kbeg + ntiles * 64);
#pragma unroll
  for (int qq = 0; qq < kPreQPW; ++qq) {
    if (qi[qq] >= n_q) continue;
    float* o = scores + ((long)b * n_q + qi[qq]) * n_kv;
    for (int t = mstart + lane; t < kend; t += 64) o[t] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
// 64-key chunks per wave of the decode kernel: about 2048 blocks (short-lived waves of two
// chunks each measured fastest: more independent streams in flight than a few long-lived
// waves), or the tuning switch when `tuned`.
// Chunks per wave: about one per 2048 block steps of the call, and at least two once the call
// has 1024 block steps (workgroups at one chunk per wave): two chunks per wave measured faster
// from there on (8 x 32768 keys: 17.1 -> 16.3 us, 16 x 32768: 28.3 -> 26.6, 1 x 262144:
// 17.2 -> 16.6, 4 x 65536: 17.2 -> 16.5, the pooled 32 x 8192: 17.9 -> 17.3 us).
static int decode_iters(long rows, int n_kv, bool tuned = true) {
  const long chunks = (n_kv + 255) / 256;  // 256-key block steps per query
  const int cpw = tuned ? g_score_cpw.load(std::memory_order_relaxed) : 0;
  long want = cpw > 0 ? cpw : (chunks * rows) / 2048;
  if (cpw <= 0 && chunks * rows >= 1024 && want < 2) want = 2;
  return want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
}

// Candidates per wave: the wave's expected share of the top-k if the chosen keys were spread
// evenly, mu = G top_k / n_kv, plus 4 standard deviations and 4, so that a wave seldom holds
// more of the top-k than it keeps (the selection then re-reads that wave's scores, and the
// select kernel lasts as long as its slowest row: at 2.5 deviations about one row in five of
// the batched decode shape needed a re-read). The fused path is taken only when the union of
// the candidates fits one select workgroup (8192 keys, or 16384 with 16 per thread: 8 x 131072
// keys, 12288 candidates, fused call 60.8 -> 58.2 us against the score kernel with the filter
// and its select) with the score kernel's own chunks per wave: with longer waves (fewer, larger
// ranges) the score kernel itself slowed down more than the fusion saved (8 x 131072: 47.4 ->
// 54.2 us at four chunks per wave), so shapes beyond that run the score and top-k kernels one
// after the other.
ScoreTopkPlan plan_score_topk(int B, int n_q, int H, int D, int n_kv, int top_k, int dtype) {
  ScoreTopkPlan p{false, 0, 0, 0, 0, false};
  const long rows = (long)B * n_q;
  if (!(D == 128 && H >= 1 && H <= 32 && (dtype == kBF16 || dtype == kF16) && n_q < 8 && rows <= 65535))
    return p;
  const long chunks = (n_kv + 255) / 256;
  // the automatic rule only, so that the workspace size does not depend on tuning switches
  for (int iters = decode_iters(rows, n_kv, false), last = iters; iters <= last; iters *= 2) {
    const long n_w = (chunks + iters - 1) / iters * 4;
    const int G = 64 * iters;
    const double mu = top_k >= n_kv ? (double)G : (double)G * top_k / n_kv;
    int m = (int)ceil(mu + 4.0 * sqrt(mu) + 4.0);
    m = m > G ? G : m;
    if (n_w <= kCandMaxWaves && n_w * m <= kCandCapWide) {
      p.ok = true;
      p.wide = n_w * m > kCandCap;
      p.iters = iters;
      p.m = m;
      p.n_w = (int)n_w;
      const size_t slots = (size_t)rows * n_w * m;
      p.cand_bytes = (slots * 8 + 255) / 256 * 256 + (size_t)rows * n_w * 16;
      return p;
    }
  }
  return p;
}

template <typename T16>
static hipError_t launch_cand_t(const void* q, const void* k, const float* w, const int* kv_len, const int* q_pos,
                                float* scores, int B, int n_q, int H, int n_kv, float scale,
                                const ScoreTopkPlan& plan, CandOut cand, hipStream_t stream) {
  const dim3 grid((unsigned)(plan.n_w / kDecWaves), (unsigned)((long)B * n_q));
  const ScoreArgs none{nullptr, 0, 0.f, 1};
#define DSA_CAND_LAUNCH(N)                                                                      \
  if (H == 32)                                                                                  \
    hipLaunchKernelGGL((index_score_decode_mfma<T16, N, true, true>), grid, dim3(256), 0, stream,  \
                       (const T16*)q, (const T16*)k, w, kv_len, q_pos, scores, n_q, H, n_kv, scale, none, cand); \
  else                                                                                          \
    hipLaunchKernelGGL((index_score_decode_mfma<T16, N, false, true>), grid, dim3(256), 0, stream, \
                       (const T16*)q, (const T16*)k, w, kv_len, q_pos, scores, n_q, H, n_kv, scale, none, cand)
  switch (plan.iters) {
    case 8: DSA_CAND_LAUNCH(8); break;
    case 4: DSA_CAND_LAUNCH(4); break;
    case 2: DSA_CAND_LAUNCH(2); break;
    default: DSA_CAND_LAUNCH(1); break;
  }
#undef DSA_CAND_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index_score_cand(const void* q, const void* k, const float* w, const int* kv_len,
                                   const int* q_pos, float* scores, int B, int n_q, int H, int n_kv, int dtype,
                                   float scale, const ScoreTopkPlan& plan, CandOut cand, hipStream_t stream) {
  if (dtype == kBF16)
    return launch_cand_t<bf16_t>(q, k, w, kv_len, q_pos, scores, B, n_q, H, n_kv, scale, plan, cand, stream);
  return launch_cand_t<f16_t>(q, k, w, kv_len, q_pos, scores, B, n_q, H, n_kv, scale, plan, cand, stream);
}

template <typename T16>
static hipError_t launch_mfma(const void* q, const void* k, const float* w, const int* kv_len,
                              const int* q_pos, float* scores, int B, int n_q, int H, int n_kv,
                              float scale, ScoreArgs sink, hipStream_t stream) {
  if (n_q >= 8) {
    const int tuned = g_score_prefill_waves.load(std::memory_order_relaxed);
    const int nwv = tuned > 0 ? tuned : kPrefillWaves;
    const int qb = nwv * kPreQPW;
    const int qblocks = (n_q + qb - 1) / qb;
    int spans = 2048 / max(1, qblocks * B);
    spans = max(1, min(spans, (n_kv + 255) / 256));
    int key_span = (n_kv + spans - 1) / spans;
    key_span = (key_span + 63) / 64 * 64;
    spans = (n_kv + key_span - 1) / key_span;
    dim3 grid(qblocks, spans, B);
#define DSA_PREFILL_LAUNCH(N, FH)                                                              \
  hipLaunchKernelGGL((index_score_prefill_mfma<T16, N, FH>), grid, dim3(N * 64), 0, stream,      \
                     (const T16*)q, (const T16*)k, w, kv_len, q_pos, scores, n_q, H, n_kv, key_span, scale, sink)
    const bool full = H == 32;
    if (nwv == 8) {
      if (full) DSA_PREFILL_LAUNCH(8, true);
      else DSA_PREFILL_LAUNCH(8, false);
    } else {
      if (full) DSA_PREFILL_LAUNCH(4, true);
      else DSA_PREFILL_LAUNCH(4, false);
    }
#undef DSA_PREFILL_LAUNCH
  } else {
    const long chunks = (n_kv + 255) / 256;  // 256-key block steps per query
    const long rows = (long)B * n_q;
    const int iters = decode_iters(rows, n_kv);
    const long xblocks = (chunks + iters - 1) / iters;
    dim3 grid((unsigned)xblocks, (unsigned)rows);
#define DSA_DECODE_LAUNCH(N)                                                                  \
  if (H == 32)                                                                                \
    hipLaunchKernelGGL((index_score_decode_mfma<T16, N, true, false>), grid, dim3(256), 0, stream, \
                       (const T16*)q, (const T16*)k, w, kv_len, q_pos, scores, n_q, H, n_kv, scale, sink, \
                       CandOut{nullptr, nullptr, 0});                                \
  else                                                                                        \
    hipLaunchKernelGGL((index_score_decode_mfma<T16, N, false, false>), grid, dim3(256), 0, stream, \
                       (const T16*)q, (const T16*)k, w, kv_len, q_pos, scores, n_q, H, n_kv, scale, sink, \
                       CandOut{nullptr, nullptr, 0})
    switch (iters) {
      case 8: DSA_DECODE_LAUNCH(8); break;
      case 4: DSA_DECODE_LAUNCH(4); break;
      case 2: DSA_DECODE_LAUNCH(2); break;
      default: DSA_DECODE_LAUNCH(1); break;
    }
#undef DSA_DECODE_LAUNCH
  }
  return hipGetLastError();
}

hipError_t launch_index_score(const void* q, const void* k, const float* w, const int* kv_len,
                              const int* q_pos, float* scores, int B, int n_q, int H, int D,
                              int n_kv, int dtype, float scale, ScoreArgs sink, hipStream_t stream) {
  const bool mfma_ok = D == 128 && H <= 32 && (dtype == kBF16 || dtype == kF16);
  if (mfma_ok) {
    if (dtype == kBF16)
      return launch_mfma<bf16_t>(q, k, w, kv_len, q_pos, scores, B, n_q, H, n_kv, scale, sink, stream);
    return launch_mfma<f16_t>(q, k, w, kv_len, q_pos, scores, B, n_q, H, n_kv, scale, sink, stream);
  }
  dim3 grid((unsigned)((n_kv + kPlainKeys - 1) / kPlainKeys), (unsigned)((long)B * n_q));
  const size_t shm = (size_t)H * D * sizeof(float);
  if (dtype == kF32)
    hipLaunchKernelGGL(index_score_plain<float>, grid, dim3(256), shm, stream, (const float*)q,
                       (const float*)k, w, kv_len, q_pos, scores, n_q, H, D, n_kv, scale, sink);
  else if (dtype == kBF16)
    hipLaunchKernelGGL(index_score_plain<bf16_t>, grid, dim3(256), shm, stream, (const bf16_t*)q,
                       (const bf16_t*)k, w, kv_len, q_pos, scores, n_q, H, D, n_kv, scale, sink);
  else
    hipLaunchKernelGGL(index_score_plain<f16_t>, grid, dim3(256), shm, stream, (const f16_t*)q,
                       (const f16_t*)k, w, kv_len, q_pos, scores, n_q, H, D, n_kv, scale, sink);
  return hipGetLastError();
}

}  // namespace dsa
