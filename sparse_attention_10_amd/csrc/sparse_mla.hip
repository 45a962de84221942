// Sparse absorbed MLA over the selected latent rows.
//
// For one query and head h, over the selected rows j (ds4 "hy3: Metal decode path" PR, GLM
// CPU oracle: cached rows are 512 latent + 64 already-rotated rope values, one softmax over
// the candidates; ik_llama_opt "MLA tensor parallelism under -sm graph": absorbed per-head
// wk_b / wv_b, so attention runs in the latent space):
//   z_j = sm_scale * q_abs[h] . row_j[0:576],  out[h] = sum_j softmax(z)_j * row_j[0:512].
// The top_k index slots of a query are cut into n_split parts. Each part is one workgroup
// that keeps a running max m, denominator l and unnormalised output o per head (online
// softmax, ds4 "Hy3 (295B)" PR, online-softmax commit); a merge pass combines the parts:
//   M = max_s m_s,  L = sum_s e^{m_s - M} l_s,  out = sum_s e^{m_s - M} o_s / L,  lse = M + ln L.
//
// MFMA kernel (bf16, 16..64 heads, 512 + {0, 64} dims): 16 selected rows at a time are
// gathered into LDS by DMA. Score waves compute S^T = C Q^T for 16 heads each, so a lane owns
// one head and four rows and the softmax needs no cross-lane work in the common case; value
// waves accumulate O^T = V^T P^T for 128 output dims of all heads, reading V^T from the
// row-major tile with ds_read_b64_tr_b16 (gfx950 transpose read), so no second copy is made.
#include "common.h"
#include "kernels.h"

#include <math.h>

#include <type_traits>

namespace dsa {

// ---------------------------------------------------------------------------------------
// plain kernel: grid (n_split, B * n_q, head groups of 8); 256 threads; rows in tiles of 16
// ---------------------------------------------------------------------------------------
constexpr int kPlainHeads = 8;
constexpr int kPlainRows = 16;
constexpr int kPlainBatch = 8;  // global loads in flight per thread while staging q and rows

template <typename T>
__global__ __launch_bounds__(256) void sparse_mla_plain(
    const T* __restrict__ qa, const T* __restrict__ lat, const int* __restrict__ idx,
    const int* __restrict__ kv_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_q, int Hm, int n_kv, int top_k,
    int d_latent, int Dc, float sm_scale, int n_split, int chunk) {
  extern __shared__ float sh[];
  float* s_q = sh;                                   // [8][Dc]
  float* s_rows = s_q + kPlainHeads * Dc;            // [16][Dc]
  float* s_z = s_rows + kPlainRows * Dc;             // [8][16]
  float* s_alpha = s_z + kPlainHeads * kPlainRows;   // [8]
  float* s_m = s_alpha + kPlainHeads;                // [8]
  float* s_l = s_m + kPlainHeads;                    // [8]
  int* s_row = reinterpret_cast<int*>(s_l + kPlainHeads);  // [16]

  const int sp = blockIdx.x;
  const int bi = blockIdx.y;
  const int h0 = blockIdx.z * kPlainHeads;
  const int nh = min(kPlainHeads, Hm - h0);
  const int b = bi / n_q;
  const int len = kv_len ? min(kv_len[b], n_kv) : n_kv;
  const int tid = threadIdx.x;

  // global loads go out kPlainBatch at a time before any is stored, so their latencies overlap
  for (int e0 = tid; e0 < kPlainHeads * Dc; e0 += 256 * kPlainBatch) {
    float v[kPlainBatch];
#pragma unroll
    for (int u = 0; u < kPlainBatch; ++u) {
      const int e = e0 + 256 * u;
      const int h = e / Dc, d = e - h * Dc;
      v[u] = (e < kPlainHeads * Dc && h < nh) ? load_as_f32(qa, ((long)bi * Hm + h0 + h) * Dc + d) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPlainBatch; ++u)
      if (e0 + 256 * u < kPlainHeads * Dc) s_q[e0 + 256 * u] = v[u];
  }
  if (tid < kPlainHeads) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  constexpr int kMaxD = 4;  // d_latent <= 1024
  float o[kPlainHeads][kMaxD];
#pragma unroll
  for (int h = 0; h < kPlainHeads; ++h)
#pragma unroll
    for (int c = 0; c < kMaxD; ++c) o[h][c] = 0.f;

  const int s0 = sp * chunk, s1 = min(top_k, s0 + chunk);
  for (int t0 = s0; t0 < s1; t0 += kPlainRows) {
    __syncthreads();
    if (tid < kPlainRows) {
      const int slot = t0 + tid;
      int r = slot < s1 ? idx[(long)bi * top_k + slot] : -1;
      s_row[tid] = (r >= 0 && r < len) ? r : -1;
    }
    __syncthreads();
    for (int e0 = tid; e0 < kPlainRows * Dc; e0 += 256 * kPlainBatch) {
      float v[kPlainBatch];
#pragma unroll
      for (int u = 0; u < kPlainBatch; ++u) {
        const int e = e0 + 256 * u;
        const int j = e / Dc, d = e - j * Dc;
        const int r = e < kPlainRows * Dc ? s_row[j] : -1;
        v[u] = r >= 0 ? load_as_f32(lat, ((long)b * n_kv + r) * Dc + d) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kPlainBatch; ++u)
        if (e0 + 256 * u < kPlainRows * Dc) s_rows[e0 + 256 * u] = v[u];
    }
    __syncthreads();
    // z for the 8 x 16 (head, row) pairs: 16 lanes per pair on consecutive dims (rows Dc
    // floats apart would put the lanes of a one-pair-per-lane loop on the same LDS banks),
    // 16 pairs per pass, the lanes' partial sums added with xor shuffles inside their group
    for (int p0 = 0; p0 < kPlainHeads * kPlainRows; p0 += 16) {
      const int pr = p0 + (tid >> 4), l = tid & 15;
      const int h = pr / kPlainRows, j = pr - h * kPlainRows;
      float acc = 0.f;
      for (int d = l; d < Dc; d += 16) acc = fmaf(s_q[h * Dc + d], s_rows[j * Dc + d], acc);
      acc += shfl_xor(acc, 8);
      acc += shfl_xor(acc, 4);
      acc += shfl_xor(acc, 2);
      acc += shfl_xor(acc, 1);
      if (l == 0) s_z[pr] = (s_row[j] >= 0 && h < nh) ? sm_scale * acc : -INFINITY;
    }
    __syncthreads();
    if (tid < kPlainHeads) {
      const int h = tid;
      float mt = -INFINITY;
      for (int j = 0; j < kPlainRows; ++j) mt = fmaxf(mt, s_z[h * kPlainRows + j]);
      const float mo = s_m[h];
      const float mn = fmaxf(mo, mt);
      float alpha = 1.f, sum = 0.f;
      if (mn != -INFINITY) {
        alpha = mo == -INFINITY ? 0.f : __expf(mo - mn);
        for (int j = 0; j < kPlainRows; ++j) {
          const float zz = s_z[h * kPlainRows + j];
          const float p = zz == -INFINITY ? 0.f : __expf(zz - mn);
          s_z[h * kPlainRows + j] = p;
          sum += p;
        }
      } else {
        for (int j = 0; j < kPlainRows; ++j) s_z[h * kPlainRows + j] = 0.f;
      }
      s_alpha[h] = alpha;
      s_m[h] = mn;
      s_l[h] = alpha * s_l[h] + sum;
    }
    __syncthreads();
    // o = alpha o + sum_j p_j row_j, row by row (each output takes the same operations in the
    // same order as a per-output loop, with one row's values and weights live at a time)
#pragma unroll
    for (int h = 0; h < kPlainHeads; ++h) {
      const float a = s_alpha[h];
#pragma unroll
      for (int c = 0; c < kMaxD; ++c) o[h][c] *= a;
    }
#pragma unroll 2
    for (int j = 0; j < kPlainRows; ++j) {
      float rv[kMaxD];
#pragma unroll
      for (int c = 0; c < kMaxD; ++c) {
        const int d = tid + 256 * c;
        rv[c] = d < d_latent ? s_rows[j * Dc + d] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < kPlainHeads; ++h) {
        const float p = s_z[h * kPlainRows + j];
#pragma unroll
        for (int c = 0; c < kMaxD; ++c) o[h][c] = fmaf(p, rv[c], o[h][c]);
      }
    }
  }
  __syncthreads();
  for (int h = 0; h < nh; ++h) {
    const long qh = (long)bi * Hm + h0 + h;
    const float m = s_m[h], l = s_l[h];
    if (n_split == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int c = 0; c < kMaxD; ++c) {
        const int d = tid + 256 * c;
        if (d < d_latent) out[qh * d_latent + d] = o[h][c] * inv;
      }
      if (lse && tid == 0) lse[qh] = l > 0.f ? m + __logf(l) : -INFINITY;
    } else {
      const long ph = ((long)bi * n_split + sp) * Hm + h0 + h;
#pragma unroll
      for (int c = 0; c < kMaxD; ++c) {
        const int d = tid + 256 * c;
        if (d < d_latent) ws_o[ph * d_latent + d] = o[h][c];
      }
      if (tid == 0) {
        ws_ml[2 * ph] = m;
        ws_ml[2 * ph + 1] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------------------
constexpr int kMlaMaxChunk = 2048;    // index slots per workgroup (LDS index buffer)

__device__ __forceinline__ f32x4 mma_bf16(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane row, lane i receives element i%4 of the 8-byte
// loads of lanes 4j + i/4 (j = 0..3), i.e. a 4x4 transpose of 16-bit values per lane quad.
// Issued through inline asm: the compiler treats the intrinsic as possibly aliasing every
// in-flight LDS DMA and would wait for all of them (draining the tile ring) before each read.
// The caller orders the reads after the tile's barrier and consumes the results only after an
// s_waitcnt lgkmcnt that has the destination registers tied to it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}
template <int OFF>
__device__ __forceinline__ i32x4 ds_read_b128_off(uint32_t base) {
  i32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ i16x4 ds_read_tr16_off(uint32_t base) {
  i16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF) : "memory");
  return v;
}
// s_waitcnt lgkmcnt(0) with the destinations of earlier LDS reads tied to it, so that they
// cannot be used before it (the reads are asm, invisible to the compiler's own waits).
__device__ __forceinline__ void tie4(i32x4& a, i32x4& b, i32x4& c, i32x4& d) {
  asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
template <int N>
__device__ __forceinline__ void tie_rest(i32x4 (&a)[N]) {
  static_assert(N >= 4 && N <= 12, "register groups");
  if constexpr (N >= 8) tie4(a[4], a[5], a[6], a[7]);
  if constexpr (N >= 12) tie4(a[8], a[9], a[10], a[11]);
  if constexpr (N % 4 == 1) asm volatile("" : "+v"(a[N - 1]));
  if constexpr (N % 4 == 2) asm volatile("" : "+v"(a[N - 2]), "+v"(a[N - 1]));
  if constexpr (N % 4 == 3) asm volatile("" : "+v"(a[N - 3]), "+v"(a[N - 2]), "+v"(a[N - 1]));
}
// all LDS reads of this wave done
template <int N>
__device__ __forceinline__ void lds_wait_all(i32x4 (&a)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : : "memory");
  tie_rest<N>(a);
}
// the reads into a[] done while the CNT reads issued after them may still be in flight (LDS
// reads of one wave complete in order)
template <int N, int CNT = N>
__device__ __forceinline__ void lds_wait_first(i32x4 (&a)[N]) {
  static_assert(CNT <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]) : "n"(CNT) : "memory");
  tie_rest<N>(a);
}
// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}
// Tile staging. A tile is 16 selected rows, row-major, each row's 16-byte chunk c stored at
// position c ^ (row & 7) (no padding; the XOR keeps both the score reads and the transpose
// reads free of bank conflicts). Tiles arrive by LDS DMA (global_load_lds_dwordx4): every
// instruction of a wave fills 64 consecutive 16-byte LDS slots, lane l the slot base + l, so
// each lane fetches whatever global chunk belongs in its slot. Slots of padding rows fetch
// from a zero row, so every wave always issues the same number of DMA instructions per tile
// and the vmcnt bookkeeping below stays exact. A 7-deep ring: two tiles are being computed on
// while five (90 KB) are in flight.
//
// Work split: waves 0..3 are score waves, one per group of 16 heads; waves 4..7 are value
// waves, one per 128 output dims, each for all heads. Wave w runs on SIMD w % 4, so every SIMD
// holds one of each. In step i the score waves compute S^T = C Q^T for tile i + 1 over all 576
// dims, run the online softmax and leave the probabilities (bf16 hi + lo parts, [head][row])
// in LDS, while the value waves accumulate O^T += V^T P^T for tile i from the probabilities
// left in the previous step (32x32x16 MFMA: 32 dims x 32 heads x the tile's 16 rows). The two
// kinds of work overlap on each SIMD: one wave's exponentials and shuffles run while the other
// keeps the matrix core busy. A barrier separates the steps.
constexpr int kTileRows = 16;
constexpr int kNst = 7;                // ring stages
constexpr float kLazyRescale = 8.0f;  // natural-log units
__device__ __attribute__((aligned(16))) const uint32_t g_zero_row[288] = {0};  // 1152 zero bytes

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ f32x16 mma32_bf16(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier after this wave's own LDS accesses have completed (lgkmcnt(0)); unlike
// __syncthreads it leaves the in-flight DMA (vmcnt) alone. The compiler-only fences keep LDS
// accesses on their side of it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // vmcnt 63 (no wait), lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// DMA blocks of a tile issued by one wave: blocks w, w + 8, ... (< nblk)
template <int NBLK>
struct DmaShare {
  static constexpr int hi = (NBLK + 7) / 8;  // waves 0 .. (NBLK % 8) - 1 (or all) issue `hi`
  static constexpr int lo = NBLK / 8;
};

// Partial-output slots (16 bytes each) per 32-head tile of one part: 4 dim quarters x 4
// dim tiles x 4 column groups x 64 lanes.
constexpr int kFragSlots = 4 * 4 * 4 * 64;
__device__ __forceinline__ int frag_slot(int pq, int ht, int n_ht, int dt, int c, int lane) {
  return (((pq * n_ht + ht) * 4 + dt) * 4 + c) * 64 + lane;
}

// The token of slot s of query row bq under the pooled indexer (KpoolSlots), or -1.
__device__ __forceinline__ int kpool_slot_token(const KpoolSlots& ks, int bq, int s, int b, int n_q, int n_kv,
                                                int len) {
  const int np = ks.kpool * ks.top_pools;
  long t;
  if (s < np) {
    const int p = ks.pool_idx[(long)bq * ks.top_pools + s / ks.kpool];
    t = p < 0 ? -1 : (long)ks.kpool * p + s % ks.kpool;
  } else {
    const long pos = ks.q_pos ? (long)ks.q_pos[bq] : (long)len - n_q + (bq - b * n_q);
    const long first = pos + 1 >= 0 ? (pos + 1) / ks.kpool * ks.kpool : -1;  // tail start
    t = first < 0 ? -1 : first + (s - np);
    if (t > pos) t = -1;
  }
  if (t < 0 || t >= len) return -1;
  const uint8_t* v = ks.packed + ((long)b * n_kv + t) * ks.row_bytes + ks.valid_off;
  const bool ok = ks.valid_f32 ? (*reinterpret_cast<const uint32_t*>(v) & 0x7fffffffu) != 0u
                               : (*reinterpret_cast<const uint16_t*>(v) & 0x7fffu) != 0u;
  return ok ? (int)t : -1;
}

// NT: the calls whose cache rows are not shared between queries (one query per sequence) read
// the tiles with the nontemporal cache policy; see the DMA issue below.
template <int DR, int NHT, int TPS, bool KP = false, bool NT = false>
__global__ __launch_bounds__(512) void sparse_mla_mfma(
    const bf16_t* __restrict__ qa, const bf16_t* __restrict__ lat, const int* __restrict__ idx,
    const int* __restrict__ kv_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_q, int Hm, int n_kv, int top_k,
    float sm_scale, int n_split, int chunk, int hsplit, KpoolSlots ks) {
  constexpr int DL = 512;
  constexpr int DC = DL + DR;
  constexpr int ROWB = DC * 2;                  // bytes per row
  constexpr int CPR = ROWB / 16;                // 16-byte chunks per row (72 or 64)
  constexpr int TILE_BYTES = kTileRows * ROWB;
  constexpr int NBLK = kTileRows * CPR / 64;    // 64-slot DMA blocks per tile (18 or 16)
  constexpr int KSW = DC / 32;                  // score k-steps (18 or 16)
  constexpr int SB = KSW % 3 == 0 ? 3 : 2;      // score k-steps per LDS batch
  constexpr int NJ = DmaShare<NBLK>::hi;
  static_assert(kTileRows * CPR % 64 == 0 && KSW % SB == 0, "tile shape");
  constexpr int SR = kTileRows * TPS;           // rows per step
  // Two tiles a step: a 7-stage ring, step it refills the stages of step it - 1 (MAXA later
  // tiles in flight when a step's tiles are due). Three tiles a step (OWN): a 6-stage ring,
  // step it refills its own stages with step it + 2's tiles (none in flight at the wait).
  constexpr bool OWN = TPS == 3;
  constexpr int NST = OWN ? 2 * TPS : kNst;     // ring stages
  constexpr int MAXA = OWN ? 0 : kNst - 3 * TPS;
  static_assert(OWN || (MAXA >= 1 && MAXA <= 4), "ring depth");

  __shared__ __attribute__((aligned(16))) uint8_t s_ring[NST * TILE_BYTES];
  __shared__ int s_idx[kMlaMaxChunk];
  // probabilities of one step's rows: [buffer][hi, lo][head][row], bf16 bits. A head's rows are
  // PS = SR + 8 values apart (SR·2 + 16 bytes): with that stride the 8-byte writes of 16 heads
  // and the 16-byte reads of 8 heads each touch distinct LDS banks (a stride of SR·2 = 32 or 64
  // bytes put 4 heads on the same banks).
  constexpr int PS = SR + 8;
  __shared__ __attribute__((aligned(16))) uint16_t s_p[2][2][64 * PS];
  __shared__ __attribute__((aligned(16))) float s_alpha[2][64];   // rescale factor per head
  __shared__ __attribute__((aligned(16))) uint32_t s_flag[2][4];  // score wave rescaled
  __shared__ float s_ml[2][64];                                   // final m, l per head

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const bool score_wave = wave < 4;
  const int hg = wave;            // score waves: head group
  const int pq = wave - 4;        // value waves: output dims 128 * pq ..
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bi = logical / n_split;
  const int sp = logical - bi * n_split;
  // with hsplit = 2 a query's 64 heads run as two workgroup rows of 32 heads (bi = 2 query +
  // half), which share the query's index row and cache
  const int bq = bi / hsplit;
  const int b = bq / n_q;
  const int len = kv_len ? min(kv_len[b], n_kv) : n_kv;
  const int s0 = sp * chunk, s1 = min(top_k, s0 + chunk);
  const int nslots = max(0, s1 - s0);
  const bool scores = score_wave && hg * 16 < Hm;
  const int head = hg * 16 + r16;

  // score waves: query operand (B of the score MFMA), lane holds head, dims 32 s + 8 g .. +8.
  // Loaded first; the slot indices go to the value waves first (slots 0 .. 255), so that the
  // two loads are in flight together rather than one after the other.
  i32x4 qreg[KSW];
  if (scores) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(qa) + ((long)bi * Hm + head) * ROWB;
#pragma unroll
    for (int s = 0; s < KSW; ++s) qreg[s] = *reinterpret_cast<const i32x4*>(qp + (4 * s + g) * 16);
  }
  for (int j = (tid + 256) & 511; j < nslots; j += 512) {
    int r;
    if constexpr (KP) r = kpool_slot_token(ks, bq, s0 + j, b, n_q, n_kv, len);
    else r = idx[(long)bq * top_k + s0 + j];
    s_idx[j] = (r >= 0 && r < len) ? r : -1;
  }
  {  // heads without a score wave keep zero probabilities
    uint4* p4 = reinterpret_cast<uint4*>(&s_p[0][0][0]);
    for (int j = tid; j < (int)(sizeof(s_p) / 16); j += 512) p4[j] = make_uint4(0u, 0u, 0u, 0u);
  }
  constexpr int n_ht = NHT;  // 32-head tiles: (Hm + 31) / 32
  // query registers ready before the first DMA, so later waits count DMAs only (with the
  // query loads left in flight here the compiler adds three full vector-memory waits to the
  // kernel, and the batched call measured 34.4-35.3 -> 38.2-38.9 us)
  wait_vmcnt<0>();
  __syncthreads();

  const uint8_t* latb = reinterpret_cast<const uint8_t*>(lat) + (long)b * n_kv * ROWB;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_zero_row);
  asm volatile("" : "+s"(zero));  // kept in scalar registers, not rebuilt from the symbol per DMA
  // the DMA share and wait counts of this wave, known uniform (scalar branches, no exec masks)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int my_blocks = wave_u < (NBLK % 8 == 0 ? 8 : NBLK % 8) ? DmaShare<NBLK>::hi : DmaShare<NBLK>::lo;
  // per-lane DMA constants: block j of this wave fills LDS slots (j*8 + wave)*64 + lane, which
  // hold chunk dma_c[j] of tile row dma_r[j]
  int dma_r[NJ], dma_c[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int slot = (j * 8 + wave) * 64 + lane;
    const int r = slot / CPR;
    dma_r[j] = r;
    dma_c[j] = ((slot - r * CPR) ^ (r & 7)) * 16;
  }
  // steps take TPS tiles; the last step's tiles past the slots are padding (zero rows, p = 0)
  const int nsteps = (nslots + SR - 1) / SR;
  const int ntiles = nsteps * TPS;
  // The cache rows of a tile's DMA slots are read from s_idx one step before the tile is
  // issued, so the DMA issue itself never waits for LDS.
  auto tile_rows = [&](int tile, int (&rows)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ts = tile * kTileRows + dma_r[j];
      rows[j] = ((j < NBLK / 8 || j * 8 + wave_u < NBLK) && ts < nslots) ? s_idx[ts] : -1;
    }
  };
  // ring stage st = tile % NST, kept by the callers as a counter (no division per step)
  auto issue = [&](int st, const int (&rows)[NJ]) {
    uint8_t* stage = s_ring + st * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int blk = j * 8 + wave_u;
      if (j < NBLK / 8 || blk < NBLK) {  // the first NBLK / 8 blocks belong to every wave
        // a select, not a branch: padding slots read the zero row
        const uintptr_t real = reinterpret_cast<uintptr_t>(latb) + (uintptr_t)((long)max(rows[j], 0) * ROWB);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(
            (rows[j] >= 0 ? real : reinterpret_cast<uintptr_t>(zero)) + dma_c[j]);
        // NT sets the nt cache-policy bit (aux bit 1): rows read once per call stream past the
        // caches' normal replacement (attention with its merge, 32 queries x 2048 rows:
        // 34.1 -> 32.9 us; 8 x 2048: 19.0 -> 18.45 us; the chunked prefill, whose 4096
        // queries share most rows through the caches, slowed 1.76 -> 1.99 ms with it)
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + blk * 1024), 16, 0, NT ? 2 : 0);
      }
    }
  };
  // waits: at most `ahead` (<= MAXA) later tiles of this wave's DMA may still be in flight
  auto wait_tiles = [&](int ahead) {
    if constexpr (OWN) {  // ahead is 0 or TPS (the prologue's second step)
      if (my_blocks == DmaShare<NBLK>::hi) {
        if (ahead >= TPS) wait_vmcnt<TPS * DmaShare<NBLK>::hi>();
        else wait_vmcnt<0>();
      } else {
        if (ahead >= TPS) wait_vmcnt<TPS * DmaShare<NBLK>::lo>();
        else wait_vmcnt<0>();
      }
      return;
    }
    if (my_blocks == DmaShare<NBLK>::hi) {
      constexpr int h = DmaShare<NBLK>::hi;
      if (ahead >= 4 && MAXA >= 4) wait_vmcnt<4 * h>();
      else if (ahead >= 3 && MAXA >= 3) wait_vmcnt<3 * h>();
      else if (ahead >= 2 && MAXA >= 2) wait_vmcnt<2 * h>();
      else if (ahead >= 1) wait_vmcnt<h>();
      else wait_vmcnt<0>();
    } else {
      constexpr int l = DmaShare<NBLK>::lo;
      if (ahead >= 4 && MAXA >= 4) wait_vmcnt<4 * l>();
      else if (ahead >= 3 && MAXA >= 3) wait_vmcnt<3 * l>();
      else if (ahead >= 2 && MAXA >= 2) wait_vmcnt<2 * l>();
      else if (ahead >= 1) wait_vmcnt<l>();
      else wait_vmcnt<0>();
    }
  };
  __syncthreads();  // s_idx and the zeroed probabilities are visible
  // Tile t goes to stage t % NST. Two tiles a step: before the first step tiles
  // [0, kNst - 2 TPS) are issued; step it then issues tiles TPS (it - 1) + kNst + h (h < TPS)
  // into the stages of step it - 1's tiles, which both kinds of wave are done with once step
  // it's barrier has passed. Three tiles a step: steps 0 and 1's tiles fill the ring before
  // the first step, and step it >= 0 issues step it + 2's tiles into its own stages, free once
  // its barrier has passed (the value waves read a step's operands at the end of the step
  // before it).
  constexpr int PRO = OWN ? 2 * TPS : kNst - 2 * TPS;  // tiles issued before the first step
  int next_rows[TPS][NJ];
  for (int p = 0; p < PRO; ++p)
    if (p < ntiles) {
      tile_rows(p, next_rows[0]);
      issue(p, next_rows[0]);  // stage p
    }
#pragma unroll
  for (int h = 0; h < TPS; ++h) tile_rows(PRO + h, next_rows[h]);

  // Score reads: row r16, chunk 4 s + g stored at (4 s + g) ^ (r16 & 7); for k-steps of one
  // parity the offset grows by 128 bytes per two steps, so two bases cover all steps.
  const int swz = r16 & 7;
  const int sc_off0 = ((g ^ swz) << 4) + r16 * ROWB;
  const int sc_off1 = (((4 + g) ^ swz) << 4) + r16 * ROWB;
  // Value reads (A operand of the 32x32x16 MFMA: lane holds dim 32 dt + l % 32, rows
  // 8 (l / 32) .. +8): transpose reads, two per dim tile (rows +0..3 and +4..7). In the 16-lane
  // group gg of lane l, lane i points at row 8 (gg / 2) + i / 4 (+4), dims d0 + 4 (i % 4) with
  // d0 = 128 pq + 32 dt + 16 (gg % 2).
  int tr_off[4][2];
  {
    const int gg = g, i = r16;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 8 * (gg >> 1) + (i >> 2) + 4 * hh;
        const int d = 128 * (pq & 3) + 32 * dt + 16 * (gg & 1) + 4 * (i & 3);
        tr_off[dt][hh] = row * ROWB + (((d >> 3) ^ (row & 7)) << 4) + (d & 7) * 2;
      }
  }

  // One step: wait for this wave's DMA of the score tiles, barrier, refill the freed stages
  // (a score wave issues its share of the refill once its first tile's operand reads are out,
  // so the issue overlaps their latency; measured a little faster in decode than issuing it
  // right after the barrier). In step it the score waves take the tiles of step u = it + 1,
  // the value waves those of step it. Both kinds of wave run the same steps (and barriers) in loops of their own, so
  // each keeps only its own state in registers. su = stage of tile TPS (it + 1).
  // Steady steps (0 <= it, TPS it <= ntiles - kNst: MAXA later tiles are in flight and all TPS
  // tiles are issued) are compiled apart from the others, without the bounds tests and the
  // case analysis of the wait count, which cost the waves scalar instructions on every step.
  auto stage_add = [](int st, int d) {  // (st + d) mod NST for -NST <= d < NST
    st += d;
    return st < 0 ? st + NST : (st >= NST ? st - NST : st);
  };
  auto step_sync = [&](int it, auto steady) {
    constexpr bool S = decltype(steady)::value;
    const int u = it + 1;  // score step
    if constexpr (OWN && S) {
      wait_vmcnt<0>();  // step u's tiles are the only ones in flight
    } else if constexpr (OWN) {
      if (u < nsteps) wait_tiles(it < 0 ? max(0, min(2 * TPS, ntiles) - TPS) : 0);
    } else if constexpr (S) {
      if (my_blocks == DmaShare<NBLK>::hi) wait_vmcnt<MAXA * DmaShare<NBLK>::hi>();
      else wait_vmcnt<MAXA * DmaShare<NBLK>::lo>();
    } else {
      // issued so far: tiles < min(TPS (it - 1) + kNst, ntiles); due: tiles < TPS (u + 1)
      if (u < nsteps) wait_tiles(max(0, min(TPS * (it - 1) + kNst, ntiles) - TPS * (u + 1)));
    }
    lds_barrier();
  };
  auto step_issue = [&](int it, int su, auto steady) {
    constexpr bool S = decltype(steady)::value;
    if constexpr (OWN) {
      if (S || it >= 0) {
#pragma unroll
        for (int h = 0; h < TPS; ++h)
          if (S || TPS * (it + 2) + h < ntiles) issue(stage_add(su, h - TPS), next_rows[h]);
      }
    } else {
#pragma unroll
      for (int h = 0; h < TPS; ++h)
        if (S || TPS * (it - 1) + kNst + h < ntiles) issue(stage_add(su, h - 2 * TPS), next_rows[h]);
    }
  };
  auto step_rows = [&](int it) {
#pragma unroll
    for (int h = 0; h < TPS; ++h) tile_rows(OWN ? TPS * (it + 3) + h : TPS * it + kNst + h, next_rows[h]);
  };
  auto step = [&](int it, int su, auto steady) {
    step_sync(it, steady);
    step_issue(it, su, steady);
    step_rows(it);
  };
  // it = -1, then the steady steps, then the rest, with su = TPS (it + 1) % NST
  auto run_steps = [&](auto&& body) {
    int it = -1, su = 0;
    body(it, su, std::false_type());
    for (++it, su = TPS; OWN ? it + 3 <= nsteps : TPS * it <= ntiles - kNst; ++it, su = stage_add(su, TPS))
      body(it, su, std::true_type());
    for (; it < nsteps; ++it, su = stage_add(su, TPS)) body(it, su, std::false_type());
  };

  // A single part writes the output rows directly. They are staged through the tile ring,
  // idle by then, one 32-head tile at a time, so that every store instruction writes 1 KB of
  // one head's row: the accumulator order would spread an instruction over 32 heads' rows, 32
  // bytes each (measured on the chunked prefill: 4.4 us to issue one workgroup's 128 KB that
  // way). Rows of the staged tile are 2048 + 16 bytes apart, so the 16-byte writes of eight
  // consecutive heads cover all LDS banks. Every wave runs the two barriers of each tile.
  constexpr int SROW = DL * 4 + 16;
  static_assert(32 * SROW <= NST * TILE_BYTES, "a 32-head output tile fits the ring");
  auto store_staged = [&](int ht) {
    lds_barrier();  // the tile's rows are in LDS
    const int nrow = min(32, Hm - 32 * ht);
    for (int k = tid; k < nrow * (DL / 4); k += 512) {
      const int r = k / (DL / 4), col = k - r * (DL / 4);
      const f32x4 v = *reinterpret_cast<const f32x4*>(s_ring + r * SROW + col * 16);
      *reinterpret_cast<f32x4*>(out + ((long)bi * Hm + 32 * ht + r) * DL + col * 4) = v;
    }
    lds_barrier();  // read before the next tile is written (the stores need not complete)
  };

  if (score_wave) {
    float m_run = -INFINITY, l_run = 0.f;
    constexpr int KH = KSW / 2;
    // the same test as `scores`, in a form the compiler sees as uniform (scalar branch)
    const bool scores_u = wave_u * 16 < Hm;
    auto score_step = [&](int it, int su, auto steady) {
      constexpr bool S = decltype(steady)::value;
      step_sync(it, steady);
      const int u = it + 1;
      const bool sc_now = scores_u && (S || u < nsteps);
      if (!sc_now) {
        step_issue(it, su, steady);
        step_rows(it);
      }
      if (sc_now) {
        const int buf = u & 1;
        int sv = -1;
        if (lane < SR) {
          const int ts = u * SR + lane;
          sv = ts < nslots ? s_idx[ts] : -1;
        }
        const uint64_t vbits = __ballot(sv >= 0);
        float z[TPS][4];
        static_for<0, TPS>([&](auto H) {
          constexpr int h = decltype(H)::value;
          const uint32_t bufa = lds_addr(s_ring + stage_add(su, h) * TILE_BYTES);
          // S^T tile h: rows 4 g + e, head r16. The k-step reads go out in two halves; the first
          // half's products run while the second half is in flight, and the k-steps feed three
          // accumulators in turn so consecutive MFMAs do not wait on each other.
          const uint32_t sb0 = bufa + sc_off0, sb1 = bufa + sc_off1;
          i32x4 ka[KH], kb[KH];
          static_for<0, KH>([&](auto K) {
            constexpr int st = decltype(K)::value;
            ka[st] = ds_read_b128_off<128 * (st >> 1)>((st & 1) ? sb1 : sb0);
          });
          static_for<0, KH>([&](auto K) {
            constexpr int st = KH + decltype(K)::value;
            kb[st - KH] = ds_read_b128_off<128 * (st >> 1)>((st & 1) ? sb1 : sb0);
          });
          if constexpr (h == 0) step_issue(it, su, steady);  // while the first tile's operands arrive
          lds_wait_first<KH>(ka);
          f32x4 sacc[3] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          static_for<0, KH>([&](auto K) {
            constexpr int st = decltype(K)::value;
            sacc[st % 3] = mma_bf16(ka[st], qreg[st], sacc[st % 3]);
          });
          lds_wait_all<KH>(kb);
          static_for<0, KH>([&](auto K) {
            constexpr int st = KH + decltype(K)::value;
            sacc[st % 3] = mma_bf16(kb[st - KH], qreg[st], sacc[st % 3]);
          });
          const uint32_t vr = (uint32_t)(vbits >> (kTileRows * h + 4 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            z[h][e] = (vr >> e) & 1u ? ((sacc[0][e] + sacc[1][e]) + sacc[2][e]) * sm_scale : -INFINITY;
        });
        // m_run is a reference max, not the exact running max: weights are exp(z - m_run) and
        // O, l are kept relative to it. It moves (and O, l are rescaled by alpha) only when a
        // score exceeds it by more than kLazyRescale, so weights stay below e^kLazyRescale
        // (harmless in fp32 and for the bf16 hi + lo split) and rescales are rare: the common
        // path needs no cross-lane reduction. m_run is equal in the four lanes of a head; each
        // lane sums the weights of its own rows (l_run) and the lanes are added at the end.
        // O / l and m_run + log(l) do not depend on the reference.
        float zl = fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3]));
#pragma unroll
        for (int h = 1; h < TPS; ++h) zl = fmaxf(zl, fmaxf(fmaxf(z[h][0], z[h][1]), fmaxf(z[h][2], z[h][3])));
        float alpha = 1.f;
        const bool rescale = __ballot(zl > m_run + kLazyRescale) != 0;
        if (rescale) {
          float mt = fmaxf(zl, shfl_xor(zl, 16));
          mt = fmaxf(mt, shfl_xor(mt, 32));
          const float m_new = fmaxf(m_run, mt);
          alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
          l_run *= alpha;
          m_run = m_new;
        }
        // p = hi + lo with both parts bf16 (round to nearest even): the value product runs
        // once per part, so the weights keep about 16 significant bits.
        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
#pragma unroll
        for (int h = 0; h < TPS; ++h) {
          float pr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pr[e] = z[h][e] == -INFINITY ? 0.f : __expf(z[h][e] - m_run);
          l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
          bf16x4 hi4, lo4;
#pragma unroll
          for (int e = 0; e < 4; ++e) hi4[e] = (__bf16)pr[e];
#pragma unroll
          for (int e = 0; e < 4; ++e) lo4[e] = (__bf16)(pr[e] - (float)hi4[e]);
          const int po = head * PS + kTileRows * h + 4 * g;
          *reinterpret_cast<bf16x4*>(&s_p[buf][0][po]) = hi4;
          *reinterpret_cast<bf16x4*>(&s_p[buf][1][po]) = lo4;
        }
        if (lane < 16) s_alpha[buf][head] = alpha;
        if (lane == 0) s_flag[buf][hg] = rescale ? 1u : 0u;
        step_rows(it);
      } else if (u < nsteps && lane == 0) {
        s_flag[u & 1][hg] = 0u;
      }
    };
    run_steps(score_step);
    // final statistics of each head
    if (scores) {
      l_run += shfl_xor(l_run, 16);
      l_run += shfl_xor(l_run, 32);
      if (g == 0) {
        s_ml[0][head] = m_run;
        s_ml[1][head] = l_run;
      }
    }
    wait_vmcnt<0>();  // no tile transfer into the ring is left in flight (the staging reuses it)
    __syncthreads();
    if (n_split == 1)
      for (int ht = 0; ht < n_ht; ++ht) store_staged(ht);
    return;
  } else {
    // O^T tiles [32 dims][32 heads], dims 128 pq + 32 dt, heads 32 ht
    f32x16 o[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][ht][e] = 0.f;
    // The value operands of step it + 1 are read at the end of step it (its tiles are in LDS
    // for the score waves) into the registers the step's products have just consumed, so a
    // step only waits for its probabilities. su = stage of the step's first tile.
    i16x4 va[TPS][4][2];
    auto read_v = [&](int su) {
      static_for<0, TPS>([&](auto H) {
        constexpr int h = decltype(H)::value;
        const uint32_t bufa = lds_addr(s_ring + stage_add(su, h) * TILE_BYTES);
        static_for<0, 4>([&](auto DT) {
          constexpr int dt = decltype(DT)::value;
          va[h][dt][0] = ds_read_tr16_off<0>(bufa + tr_off[dt][0]);
          va[h][dt][1] = ds_read_tr16_off<0>(bufa + tr_off[dt][1]);
        });
      });
    };
    const uint32_t p_off = ((lane & 31) * PS + 8 * (lane >> 5)) * 2;
    auto value_step = [&](int it, int su, auto steady) {
      constexpr bool S = decltype(steady)::value;
      step(it, su, steady);  // its lgkmcnt(0) wait completes the reads into va
      // With three tiles a step, the value wave yields its SIMD for about 640 cycles after the
      // barrier, so that the score wave on the same SIMD (waves w and w + 4 share one) issues
      // its products before the value wave's 48 queue ahead of them on the matrix core; the
      // softmax, which waits for those products, then starts earlier. Measured on the chunked
      // prefill (4096 x 2048 slots, A/B on one box): 1.73-1.76 ms without, 1.71-1.73 with 512
      // cycles, 1.69-1.72 with 640, 1.70-1.72 with 768. Two tiles a step gained nothing.
      if constexpr (TPS == 3) __builtin_amdgcn_s_sleep(10);
      if (S || it >= 0) {
        const int buf = it & 1;
        const uint4 fl = *reinterpret_cast<const uint4*>(s_flag[buf]);
        if ((fl.x | fl.y | fl.z | fl.w) != 0u) {  // uniform: some head group moved its reference
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) {
            const float a = s_alpha[buf][32 * ht + (lane & 31)];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int e = 0; e < 16; ++e) o[dt][ht][e] *= a;
          }
        }
        // B operands: P^T [16 rows of tile h][32 heads], lane holds head 32 ht + l % 32, rows
        // 16 h + 8 (l / 32) ..
        const uint32_t pbase = lds_addr(&s_p[buf][0][0]) + p_off;
        constexpr int PHL = 64 * PS * 2;  // bytes between the hi and lo parts
        constexpr int PHT = 32 * PS * 2;  // bytes between the two head tiles
        static_for<0, TPS>([&](auto H) {
          constexpr int h = decltype(H)::value;
          constexpr int PH = kTileRows * 2 * h;  // bytes to tile h's rows
          i32x4 pb[4];
          pb[0] = ds_read_b128_off<PH>(pbase);
          pb[1] = ds_read_b128_off<PH + PHL>(pbase);
          pb[2] = ds_read_b128_off<PH + PHT>(pbase);
          pb[3] = ds_read_b128_off<PH + PHT + PHL>(pbase);
          lds_wait_all<4>(pb);
          asm volatile("" : "+v"(va[h][0][0]), "+v"(va[h][0][1]), "+v"(va[h][1][0]), "+v"(va[h][1][1]),
                       "+v"(va[h][2][0]), "+v"(va[h][2][1]), "+v"(va[h][3][0]), "+v"(va[h][3][1]));
          // all hi-part products first, then the lo parts: the two products into one
          // accumulator are eight MFMAs apart, so none waits for the previous one's result
          i32x4 av[4];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            av[dt] = __builtin_bit_cast(i32x4, __builtin_shufflevector(va[h][dt][0], va[h][dt][1], 0, 1, 2, 3, 4,
                                                                       5, 6, 7));
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int ht = 0; ht < 2; ++ht)
                if (ht < n_ht) o[dt][ht] = mma32_bf16(av[dt], pb[2 * ht + hl], o[dt][ht]);
        });
      }
      if (S || it + 1 < nsteps) read_v(su);  // step it + 1
    };
    run_steps(value_step);
    wait_vmcnt<0>();
    __syncthreads();  // the score waves' statistics are in s_ml
    // lane holds O^T[32 dt + 8 (i / 4) + 4 (l / 32) + i % 4][32 ht + l % 32], i < 16
    if (n_split == 1) {
#pragma unroll
      for (int ht = 0; ht < n_ht; ++ht) {
        const int hr = lane & 31;  // row of the staged tile
        const int h = 32 * ht + hr;
        if (h < Hm) {
          const float m = s_ml[0][h], l = s_ml[1][h];
          const float scale = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int d = 128 * pq + 32 * dt + 8 * c + 4 * (lane >> 5);
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = o[dt][ht][4 * c + e] * scale;
              *reinterpret_cast<f32x4*>(s_ring + hr * SROW + d * 4) = v;
            }
          if (lse && pq == 0 && lane < 32) lse[(long)bi * Hm + h] = l > 0.f ? m + __logf(l) : -INFINITY;
        }
        store_staged(ht);
      }
      return;
    }
    // Partial outputs in fragment order (see mla_merge_frag): every store instruction of the
    // wave writes 1 KB contiguous, where the [head][dim] order would spread it over 32 rows
    // 2 KB apart.
#pragma unroll
    for (int ht = 0; ht < n_ht; ++ht) {
      const int h = 32 * ht + (lane & 31);
      if (h >= Hm) continue;
      const long ph = ((long)bi * n_split + sp) * Hm + h;
      if (pq == 0 && lane < 32) {
        ws_ml[2 * ph] = s_ml[0][h];
        ws_ml[2 * ph + 1] = s_ml[1][h];
      }
      float* blk = ws_o + ((long)bi * n_split + sp) * (n_ht * kFragSlots) * 4;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[dt][ht][4 * c + e];
          *reinterpret_cast<f32x4*>(blk + frag_slot(pq, ht, n_ht, dt, c, lane) * 4) = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------------------
// merge of the MFMA kernel's partials, stored per part in fragment order: 16-byte slot
// ((((pq * n_ht + ht) * 4 + dt) * 4 + c) * 64 + lane) holds output dims
// d = 128 pq + 32 dt + 8 c + 4 (lane / 32) .. +3 of head 32 ht + lane % 32. One thread per
// slot; consecutive threads read consecutive slots of every part. (Nontemporal loads of the
// partials here measured 34.1 -> 33.6 us for the batched decode's attention with its merge
// alone, but 32.9 -> 34.3 us beside the attention kernel's nontemporal tile reads, so they stay
// default; nontemporal stores of the partials were slower as well.)
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_merge_frag(const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_ml,
                                                      float* __restrict__ out, float* __restrict__ lse,
                                                      int Hm, int n_ht, int n_split, long total) {
  const long gid = (long)xcd_remap(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (gid >= total) return;
  const int per = n_ht * kFragSlots;  // slots per part
  const long bi = gid / per;
  const int s = (int)(gid - bi * per);
  const int lane = s & 63, c = (s >> 6) & 3, dt = (s >> 8) & 3, hq = s >> 10;
  const int ht = hq % n_ht, pq = hq / n_ht;
  const int h = 32 * ht + (lane & 31);
  if (h >= Hm) return;
  const int d = 128 * pq + 32 * dt + 8 * c + 4 * (lane >> 5);
  constexpr int SB = 8;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_split; s0 += SB) {
    float m[SB], l[SB];
    f32x4 v[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const long part = bi * n_split + s0 + j;
      const bool in = s0 + j < n_split;
      m[j] = in ? ws_ml[2 * (part * Hm + h)] : -INFINITY;
      l[j] = in ? ws_ml[2 * (part * Hm + h) + 1] : 0.f;
      v[j] = in ? *reinterpret_cast<const f32x4*>(ws_o + (part * per + s) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < SB; ++j) mb = fmaxf(mb, m[j]);
    if (mb == -INFINITY) continue;
    const float r = M == -INFINITY ? 0.f : __expf(M - mb);
    L *= r;
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] *= r;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if (m[j] == -INFINITY) continue;
      const float f = __expf(m[j] - mb);
      L = fmaf(f, l[j], L);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(f, v[j][k], acc[k]);
    }
    M = mb;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] *= inv;
  *reinterpret_cast<f32x4*>(out + (bi * Hm + h) * 512 + d) = acc;
  if (lse && d == 0) lse[bi * Hm + h] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// The same merge with PG threads per slot, for calls whose slots alone would give too few
// workgroups (few queries, many parts): thread group g of a block (SPB = 256 / PG consecutive
// slots) takes parts [g n_split / PG, (g + 1) n_split / PG), and group 0 combines the groups'
// (M, L, acc) through LDS. Long decode (8 queries, 16 parts of 128 slots): 256 workgroups,
// attention with its merge 22.0 us; 1024 workgroups of four groups 19.0 us (eight groups:
// 21.2 us). The batched decode's 1024 workgroups gain nothing from groups (two: 34.8 -> 35.9).
template <int PG>
__global__ __launch_bounds__(256) void mla_merge_frag_g(const float* __restrict__ ws_o,
                                                        const float* __restrict__ ws_ml,
                                                        float* __restrict__ out, float* __restrict__ lse,
                                                        int Hm, int n_ht, int n_split, long total) {
  constexpr int SPB = 256 / PG;
  __shared__ f32x4 s_acc[PG][SPB];
  __shared__ float s_m[PG][SPB], s_l[PG][SPB];
  const int grp = threadIdx.x / SPB, ls = threadIdx.x - grp * SPB;
  const long gid = (long)xcd_remap(blockIdx.x, gridDim.x) * SPB + ls;
  const int per = n_ht * kFragSlots;  // slots per part
  const long bi = gid / per;
  const int s = (int)(gid - bi * per);
  const int lane = s & 63, c = (s >> 6) & 3, dt = (s >> 8) & 3, hq = s >> 10;
  const int ht = hq % n_ht, pq = hq / n_ht;
  const int h = 32 * ht + (lane & 31);
  const bool live = gid < total && h < Hm;
  const int d = 128 * pq + 32 * dt + 8 * c + 4 * (lane >> 5);
  const int p0 = grp * n_split / PG, p1 = (grp + 1) * n_split / PG;
  constexpr int SB = 8;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    for (int s0 = p0; s0 < p1; s0 += SB) {
      float m[SB], l[SB];
      f32x4 v[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const long part = bi * n_split + s0 + j;
        const bool in = s0 + j < p1;
        m[j] = in ? ws_ml[2 * (part * Hm + h)] : -INFINITY;
        l[j] = in ? ws_ml[2 * (part * Hm + h) + 1] : 0.f;
        v[j] = in ? *reinterpret_cast<const f32x4*>(ws_o + (part * per + s) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < SB; ++j) mb = fmaxf(mb, m[j]);
      if (mb == -INFINITY) continue;
      const float r = M == -INFINITY ? 0.f : __expf(M - mb);
      L *= r;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] *= r;
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        if (m[j] == -INFINITY) continue;
        const float f = __expf(m[j] - mb);
        L = fmaf(f, l[j], L);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = fmaf(f, v[j][k], acc[k]);
      }
      M = mb;
    }
  }
  s_m[grp][ls] = M;
  s_l[grp][ls] = L;
  s_acc[grp][ls] = acc;
  __syncthreads();
  if (grp != 0 || !live) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int g = 0; g < PG; ++g) Mt = fmaxf(Mt, s_m[g][ls]);
  float Lt = 0.f;
  f32x4 at = {0.f, 0.f, 0.f, 0.f};
  if (Mt != -INFINITY) {
#pragma unroll
    for (int g = 0; g < PG; ++g) {
      const float mg = s_m[g][ls];
      if (mg == -INFINITY) continue;
      const float f = __expf(mg - Mt);
      Lt = fmaf(f, s_l[g][ls], Lt);
      const f32x4 ag = s_acc[g][ls];
#pragma unroll
      for (int k = 0; k < 4; ++k) at[k] = fmaf(f, ag[k], at[k]);
    }
  }
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) at[k] *= inv;
  *reinterpret_cast<f32x4*>(out + (bi * Hm + h) * 512 + d) = at;
  if (lse && d == 0) lse[bi * Hm + h] = Lt > 0.f ? Mt + __logf(Lt) : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// merge: one thread per 4 output values (d_latent % 4 == 0), or per value otherwise.
// Consecutive threads read consecutive 16-byte pieces of each split's partial output.
// ---------------------------------------------------------------------------------------
template <int VEC>
__global__ __launch_bounds__(256) void mla_merge(const float* __restrict__ ws_o,
                                                 const float* __restrict__ ws_ml,
                                                 float* __restrict__ out, float* __restrict__ lse,
                                                 int Hm, int n_split, int dv, long total) {
  typedef __attribute__((__vector_size__(VEC * sizeof(float)))) float fv;
  // over (query, head, dims / VEC); XCD-aware order, so a query's merge runs on the XCD whose
  // L2 received that query's partial outputs from the attention kernel
  const long gid = (long)xcd_remap(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (gid >= total) return;
  const long qh = gid / dv;
  const int dq = (int)(gid - qh * dv);
  const long bi = qh / Hm;
  const int h = (int)(qh - bi * Hm);
  const long p0 = bi * n_split * Hm + h;  // partial (bi, s = 0, h); split stride Hm
  // splits in batches of 8 whose loads are all issued before use; a running max rescales
  constexpr int SB = 8;
  float M = -INFINITY, L = 0.f;
  fv acc = {};
  for (int s0 = 0; s0 < n_split; s0 += SB) {
    float m[SB], l[SB];
    fv v[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      const long ph = p0 + (long)(s0 + j) * Hm;
      const bool in = s0 + j < n_split;
      m[j] = in ? ws_ml[2 * ph] : -INFINITY;
      l[j] = in ? ws_ml[2 * ph + 1] : 0.f;
      v[j] = in ? *reinterpret_cast<const fv*>(ws_o + (ph * dv + dq) * VEC) : fv{};
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < SB; ++j) mb = fmaxf(mb, m[j]);
    if (mb == -INFINITY) continue;
    const float r = M == -INFINITY ? 0.f : __expf(M - mb);
    L *= r;
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] *= r;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if (m[j] == -INFINITY) continue;
      const float f = __expf(m[j] - mb);
      L = fmaf(f, l[j], L);
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[k] = fmaf(f, v[j][k], acc[k]);
    }
    M = mb;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) acc[j] *= inv;
  *reinterpret_cast<fv*>(out + (qh * dv + dq) * VEC) = acc;
  if (lse && dq == 0) lse[qh] = L > 0.f ? M + __logf(L) : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

std::atomic<int> g_mla_tiles_per_step{0};
std::atomic<int> g_mla_head_split{0};

// Workgroup rows per query of the MFMA kernel: 2 (32 heads each) when 64 heads would leave
// at least half of the 256 CUs without a workgroup, else 1. Partials keep the same bytes.
static int mla_head_split(int Hm, long rows, int n_split, int tuned) {
  if (Hm != 64 || tuned == 1) return 1;
  if (tuned == 2) return 2;
  return rows * n_split <= 128 ? 2 : 1;
}  // measured faster on every workload (fewer barrier steps)

int mla_auto_splits(int B, int n_q, int top_k) {
  const long rows = (long)B * n_q;
  // at most one workgroup per CU: a second round of workgroups costs most of a first (decode
  // attention with its merge, 24 queries x 2048 slots: 45.8 us at 11 parts, 33.1 us at 10;
  // 48 queries: 62.9 us at 6 parts, 43.2 us at 5)
  long s = 256 / rows;
  // parts shorter than 400 slots: about three workgroups per four CUs instead. A short part's
  // fixed costs (slot and query loads, the partial stores and their merge) weigh more than the
  // idle CUs (attention with its merge, 2048 slots: 24 queries 33.0 -> 30.4 us at 8 parts
  // instead of 10, 16 queries 26.9 -> 25.9 at 12 instead of 16; 32 queries 34.2 -> 33.7 at 6
  // instead of 8, the same decode step within noise)
  if (s >= 1 && top_k / s < 400 && 192 / rows >= 1) s = 192 / rows;
  // at least 128 slots per part; short selections may still take up to 4 parts of 16 slots
  // (one tile each), which cuts the serial row fetches of a single workgroup
  long max_s = top_k / 128;
  if (max_s < 4) max_s = top_k / 16 < 4 ? top_k / 16 : 4;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  const long min_s = (top_k + kMlaMaxChunk - 1) / kMlaMaxChunk;
  if (s < min_s) s = min_s;
  if (s < 1) s = 1;
  return (int)s;
}

size_t mla_workspace_bytes(int B, int n_q, int Hm, int top_k, int d_latent, int n_split) {
  (void)top_k;
  if (n_split <= 1) return 0;
  const size_t parts = (size_t)B * n_q * n_split;
  const size_t hpad = (size_t)(Hm + 31) / 32 * 32;  // the MFMA kernel's fragment order pads heads to 32
  return align256(parts * hpad * d_latent * sizeof(float)) + align256(parts * Hm * 2 * sizeof(float));
}

bool mla_mfma_supported(int Hm, int d_latent, int d_rope, int dtype) {
  return dtype == kBF16 && Hm % 16 == 0 && Hm <= 64 && d_latent == 512 && (d_rope == 64 || d_rope == 0);
}

hipError_t launch_sparse_mla(const void* q_abs, const void* latent, const int* idx,
                             const int* kv_len, float* out, float* lse, int B, int n_q, int Hm,
                             int n_kv, int top_k, int d_latent, int d_rope, float sm_scale,
                             int dtype, int n_split, void* workspace, hipStream_t stream,
                             const KpoolSlots* kp) {
  const int chunk = (top_k + n_split - 1) / n_split;
  const long rows = (long)B * n_q;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (n_split > 1) {
    const size_t hpad = (size_t)(Hm + 31) / 32 * 32;
    ws_o = reinterpret_cast<float*>(workspace);
    ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                     align256((size_t)rows * n_split * hpad * d_latent * sizeof(float)));
  }
  // the tuning switches are read once, so the attention kernel and its merge agree on the layout
  const int hs = mla_head_split(Hm, rows, n_split, g_mla_head_split.load(std::memory_order_relaxed));
  // tiles per step: three for parts of at least 1024 slots (43 barrier steps instead of 64 for
  // 2048 slots: 1.81-1.83 -> 1.75-1.77 ms for the chunked prefill of 4096 queries), else two
  // (decode parts of 128 or 256 slots would end in a mostly empty 48-row step)
  const int tuned_tps = g_mla_tiles_per_step.load(std::memory_order_relaxed);
  const int tps = tuned_tps ? tuned_tps : (chunk >= 1024 ? 3 : 2);
  if (mla_mfma_supported(Hm, d_latent, d_rope, dtype)) {
    const int Hk = Hm / hs;  // heads per workgroup row; the [query][head] arrays are read as [query * hs][Hk]
    const unsigned blocks = (unsigned)(rows * hs * n_split);
    // the pooled-indexer slots (kp) run with two tiles per step whatever the tuning
    // one query per sequence: no row is shared between the call's workgroups of different
    // queries, so the two-tile kernels stream the rows (NT)
    const bool nt = n_q == 1;
    auto kernel = kp
        ? (nt ? (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 2, true, true> : sparse_mla_mfma<64, 1, 2, true, true>)
                              : (Hk > 32 ? sparse_mla_mfma<0, 2, 2, true, true> : sparse_mla_mfma<0, 1, 2, true, true>))
              : (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 2, true> : sparse_mla_mfma<64, 1, 2, true>)
                              : (Hk > 32 ? sparse_mla_mfma<0, 2, 2, true> : sparse_mla_mfma<0, 1, 2, true>)))
        : tps == 2 && nt
        ? (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 2, false, true> : sparse_mla_mfma<64, 1, 2, false, true>)
                        : (Hk > 32 ? sparse_mla_mfma<0, 2, 2, false, true> : sparse_mla_mfma<0, 1, 2, false, true>))
        : tps == 3
        ? (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 3> : sparse_mla_mfma<64, 1, 3>)
                        : (Hk > 32 ? sparse_mla_mfma<0, 2, 3> : sparse_mla_mfma<0, 1, 3>))
        : tps == 2
        ? (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 2> : sparse_mla_mfma<64, 1, 2>)
                        : (Hk > 32 ? sparse_mla_mfma<0, 2, 2> : sparse_mla_mfma<0, 1, 2>))
        : (d_rope == 64 ? (Hk > 32 ? sparse_mla_mfma<64, 2, 1> : sparse_mla_mfma<64, 1, 1>)
                        : (Hk > 32 ? sparse_mla_mfma<0, 2, 1> : sparse_mla_mfma<0, 1, 1>));
    const KpoolSlots ks = kp ? *kp : KpoolSlots{nullptr, nullptr, 0, 0, 0, 0, 1, nullptr};
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(512), 0, stream, (const bf16_t*)q_abs, (const bf16_t*)latent,
                       idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hk, n_kv, top_k, sm_scale, n_split, chunk, hs, ks);
  } else {
    if (kp) return hipErrorInvalidValue;  // the pooled-indexer slots exist on the MFMA kernel only
    const int Dc = d_latent + d_rope;
    dim3 grid(n_split, (unsigned)rows, (Hm + kPlainHeads - 1) / kPlainHeads);
    const size_t shm = (size_t)(kPlainHeads * Dc + kPlainRows * Dc + kPlainHeads * kPlainRows +
                                3 * kPlainHeads) * sizeof(float) + kPlainRows * sizeof(int);
    if (shm > 65536) {
      hipError_t e = dtype == kF32
          ? hipFuncSetAttribute((const void*)sparse_mla_plain<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm)
          : hipFuncSetAttribute((const void*)sparse_mla_plain<bf16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
      if (e != hipSuccess) return e;
    }
    if (dtype == kF32)
      hipLaunchKernelGGL(sparse_mla_plain<float>, grid, dim3(256), shm, stream, (const float*)q_abs,
                         (const float*)latent, idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hm, n_kv, top_k,
                         d_latent, Dc, sm_scale, n_split, chunk);
    else
      hipLaunchKernelGGL(sparse_mla_plain<bf16_t>, grid, dim3(256), shm, stream, (const bf16_t*)q_abs,
                         (const bf16_t*)latent, idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hm, n_kv, top_k,
                         d_latent, Dc, sm_scale, n_split, chunk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  if (mla_mfma_supported(Hm, d_latent, d_rope, dtype)) {
    const int n_ht = (Hm / hs + 31) / 32;
    const long total = rows * hs * n_ht * kFragSlots;
    // thread groups per slot: doubled while the merge has fewer than 1024 workgroups and every
    // group keeps two parts or more
    int pg = 1;
    while (pg < 4 && (total + 255) / 256 * pg < 1024 && n_split >= 4 * pg) pg *= 2;
    const unsigned nb = (unsigned)((total * pg + 255) / 256);
    if (pg == 4)
      hipLaunchKernelGGL(mla_merge_frag_g<4>, dim3(nb), dim3(256), 0, stream, ws_o, ws_ml, out, lse, Hm / hs, n_ht,
                         n_split, total);
    else if (pg == 2)
      hipLaunchKernelGGL(mla_merge_frag_g<2>, dim3(nb), dim3(256), 0, stream, ws_o, ws_ml, out, lse, Hm / hs, n_ht,
                         n_split, total);
    else
      hipLaunchKernelGGL(mla_merge_frag, dim3(nb), dim3(256), 0, stream, ws_o, ws_ml, out, lse, Hm / hs, n_ht,
                         n_split, total);
  } else if (d_latent % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
    const long total = rows * Hm * (d_latent / 4);
    hipLaunchKernelGGL(mla_merge<4>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, ws_o, ws_ml,
                       out, lse, Hm, n_split, d_latent / 4, total);
  } else {
    const long total = rows * Hm * d_latent;
    hipLaunchKernelGGL(mla_merge<1>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, ws_o, ws_ml,
                       out, lse, Hm, n_split, d_latent, total);
  }
  return hipGetLastError();
}

}  // namespace dsa
