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
// MFMA kernel (bf16, 16..64 heads, 512 + {0, 64} dims): 32 selected rows at a time are
// gathered with coalesced 16-byte loads into LDS (row-major, padded rows). Each wave owns 16
// heads. Scores are computed transposed, S^T = C Q^T, so a lane owns one head and eight rows:
// the softmax statistics of a head live in one lane column and the probabilities are already
// in the B-operand layout of the value product O^T = V^T P^T. V^T is read from the row-major
// tile with ds_read_b64_tr_b16 (gfx950 transpose read), so no second copy is made.
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

  for (int e = tid; e < kPlainHeads * Dc; e += 256) {
    const int h = e / Dc, d = e - h * Dc;
    s_q[e] = h < nh ? load_as_f32(qa, ((long)bi * Hm + h0 + h) * Dc + d) : 0.f;
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
    for (int e = tid; e < kPlainRows * Dc; e += 256) {
      const int j = e / Dc, d = e - j * Dc;
      const int r = s_row[j];
      s_rows[e] = r >= 0 ? load_as_f32(lat, ((long)b * n_kv + r) * Dc + d) : 0.f;
    }
    __syncthreads();
    if (tid < kPlainHeads * kPlainRows) {
      const int h = tid / kPlainRows, j = tid - h * kPlainRows;
      float z = -INFINITY;
      if (s_row[j] >= 0 && h < nh) {
        float acc = 0.f;
        for (int d = 0; d < Dc; ++d) acc = fmaf(s_q[h * Dc + d], s_rows[j * Dc + d], acc);
        z = sm_scale * acc;
      }
      s_z[tid] = z;
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
#pragma unroll
    for (int c = 0; c < kMaxD; ++c) {
      const int d = tid + 256 * c;
      if (d >= d_latent) break;
#pragma unroll
      for (int h = 0; h < kPlainHeads; ++h) {
        float acc = o[h][c] * s_alpha[h];
        for (int j = 0; j < kPlainRows; ++j) acc = fmaf(s_z[h * kPlainRows + j], s_rows[j * Dc + d], acc);
        o[h][c] = acc;
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
constexpr int kMlaRows = 32;          // rows per LDS tile
constexpr int kMlaMaxChunk = 2048;    // index slots per workgroup (LDS index buffer)

__device__ __forceinline__ f32x4 mma_bf16(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane row, lane i receives element i%4 of the 8-byte
// loads of lanes 4j + i/4 (j = 0..3), i.e. a 4x4 transpose of 16-bit values per lane quad.
// Issued through inline asm: the compiler treats the intrinsic as possibly aliasing every
// in-flight LDS DMA and would wait for all of them (draining the tile ring) before each read.
// The caller orders the reads after the tile's barrier and consumes the results only after
// tr_wait(), which ties the destination registers to an s_waitcnt lgkmcnt(0).
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
// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}
// Tie 16-byte results to an lgkmcnt(0) wait: they cannot be used before it.
__device__ __forceinline__ void lds_wait4(i32x4& a, i32x4& b, i32x4& c, i32x4& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : : "memory");
}
__device__ __forceinline__ void lds_wait6(i32x4& a, i32x4& b, i32x4& c, i32x4& d, i32x4& e, i32x4& f) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f) : : "memory");
}

// Tile staging. A tile is 32 selected rows, row-major, each row's 16-byte chunk c stored at
// position c ^ (row & 7) (no padding; the XOR keeps both the score reads and the transpose
// reads free of bank conflicts). Tiles arrive by LDS DMA (global_load_lds_dwordx4): every
// instruction of a wave fills 64 consecutive 16-byte LDS slots, lane l the slot base + l, so
// each lane fetches whatever global chunk belongs in its slot. Slots of padding rows fetch
// from a zero row, so every wave always issues the same number of DMA instructions per tile
// and the vmcnt bookkeeping below stays exact. A 3-deep ring keeps two tiles (72 KB) in flight
// per workgroup while the third is consumed.
//
// Work split: 8 waves, two per group of 16 heads. The pair splits the score contraction (each
// wave 288 of the 576 dims; partial scores are exchanged through LDS and summed) and the
// value product (each wave 256 of the 512 output dims). Both waves of a pair then hold the
// same scores and run the same softmax, and each keeps only half of the query and of the
// output accumulators, so two waves fit per SIMD.
constexpr int kStages = 3;
constexpr float kLazyRescale = 8.0f;  // natural-log units
__device__ __attribute__((aligned(16))) const uint32_t g_zero_row[288] = {0};  // 1152 zero bytes

typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier without the release fence of __syncthreads (which would wait for every
// outstanding DMA); the compiler-only fences keep LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// The same after this wave's own LDS writes have completed (lgkmcnt(0), vmcnt untouched).
__device__ __forceinline__ void lds_write_barrier() {
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

template <int DR>
__global__ __launch_bounds__(512) void sparse_mla_mfma(
    const bf16_t* __restrict__ qa, const bf16_t* __restrict__ lat, const int* __restrict__ idx,
    const int* __restrict__ kv_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_q, int Hm, int n_kv, int top_k,
    float sm_scale, int n_split, int chunk) {
  constexpr int DL = 512;
  constexpr int DC = DL + DR;
  constexpr int ROWB = DC * 2;                  // bytes per row
  constexpr int CPR = ROWB / 16;                // 16-byte chunks per row (72 or 64)
  constexpr int TILE_BYTES = kMlaRows * ROWB;
  constexpr int NBLK = kMlaRows * CPR / 64;     // 64-slot DMA blocks per tile (36 or 32)
  constexpr int KSW = DC / 64;                  // score k-steps per wave (9 or 8)
  constexpr int NTW = DL / 32;                  // 16-dim output tiles per wave (16)
  constexpr int SB = KSW % 3 == 0 ? 3 : 2;      // score k-steps per LDS batch
  static_assert(kMlaRows * CPR % 64 == 0 && KSW % SB == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kStages * TILE_BYTES];
  __shared__ int s_idx[kMlaMaxChunk];
  __shared__ __attribute__((aligned(16))) f32x4 s_xch[8][2][64];  // partial scores per wave

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave & 3, hf = wave >> 2;      // head group, half
  const int g = lane >> 4, r16 = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bi = logical / n_split;
  const int sp = logical - bi * n_split;
  const int b = bi / n_q;
  const int len = kv_len ? min(kv_len[b], n_kv) : n_kv;
  const int s0 = sp * chunk, s1 = min(top_k, s0 + chunk);
  const int nslots = max(0, s1 - s0);
  const bool computes = hg * 16 < Hm;
  const int head = hg * 16 + r16;

  for (int j = tid; j < nslots; j += 512) {
    const int r = idx[(long)bi * top_k + s0 + j];
    s_idx[j] = (r >= 0 && r < len) ? r : -1;
  }

  // query operand (B of the score MFMA) for this wave's half of the dims:
  // lane holds head, dims 32 * (hf * KSW + s) + 8 * g .. +8
  i32x4 qreg[KSW];
  if (computes) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(qa) + ((long)bi * Hm + head) * ROWB;
#pragma unroll
    for (int s = 0; s < KSW; ++s)
      qreg[s] = *reinterpret_cast<const i32x4*>(qp + (4 * (hf * KSW + s) + g) * 16);
  }
  f32x4 o[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  wait_vmcnt<0>();  // query registers ready before the first DMA, so later waits count DMAs only
  __syncthreads();

  const uint8_t* latb = reinterpret_cast<const uint8_t*>(lat) + (long)b * n_kv * ROWB;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(g_zero_row);
  constexpr int NJ = DmaShare<NBLK>::hi;
  const int my_blocks = wave < (NBLK % 8 == 0 ? 8 : NBLK % 8) ? DmaShare<NBLK>::hi : DmaShare<NBLK>::lo;
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
  auto issue = [&](int tile) {
    uint8_t* stage = s_ring + (tile % kStages) * TILE_BYTES;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int blk = j * 8 + wave;
      if (blk < NBLK) {
        const int ts = tile * kMlaRows + dma_r[j];
        const int row = ts < nslots ? s_idx[ts] : -1;
        const uint8_t* src = (row >= 0 ? latb + (long)row * ROWB : zero) + dma_c[j];
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + blk * 1024), 16, 0, 0);
      }
    }
  };
  // waits: at most `ahead` later tiles of this wave's DMA may still be in flight
  auto wait_tile = [&](int ahead) {
    if (my_blocks == DmaShare<NBLK>::hi) {
      if (ahead >= 1) wait_vmcnt<DmaShare<NBLK>::hi>();
      else wait_vmcnt<0>();
    } else {
      if (ahead >= 1) wait_vmcnt<DmaShare<NBLK>::lo>();
      else wait_vmcnt<0>();
    }
  };
  static_assert(kStages == 3, "wait_tile assumes one tile ahead");

  const int ntiles = (nslots + kMlaRows - 1) / kMlaRows;
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < ntiles) issue(p);

  // Per-lane LDS offsets inside a tile. Score reads: rows r16 and 16 + r16 (same r & 7), chunk
  // 4 * S + g with S = hf * KSW + s stored at (4S + g) ^ (r & 7); for k-steps of one parity the
  // offset grows by 128 bytes per two steps, so two bases cover all steps (immediates do the
  // rest). Transpose reads: rows 4g + r16/4 (+16), chunk 2 * T + (r16 % 4) / 2 with
  // T = 16 * hf + t; four bases by t % 4, 128 bytes per four tiles.
  const int swz = r16 & 7;
  const int sc_off0 = (((4 * (hf * KSW + 0) + g) ^ swz) << 4) + r16 * ROWB;
  const int sc_off1 = (((4 * (hf * KSW + 1) + g) ^ swz) << 4) + r16 * ROWB;
  const int tr_row = 4 * g + (r16 >> 2);
  const int tr_x = tr_row & 7;
  const int tr_c = (r16 & 3) >> 1;
  int tr_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) tr_off[j] = tr_row * ROWB + (((2 * (16 * hf + j) + tr_c) ^ tr_x) << 4) + (r16 & 1) * 8;

  for (int tile = 0; tile < ntiles; ++tile) {
    wait_tile(min(kStages - 2, ntiles - 1 - tile));
    lds_barrier();
    if (tile + kStages - 1 < ntiles) issue(tile + kStages - 1);
    const uint32_t bufa = lds_addr(s_ring + (tile % kStages) * TILE_BYTES);
    // row validity of this tile: bit r set when tile row r holds a selected cache row
    int sv = -1;
    if (lane < kMlaRows) {
      const int ts = tile * kMlaRows + lane;
      sv = ts < nslots ? s_idx[ts] : -1;
    }
    const uint32_t vbits = (uint32_t)__ballot(sv >= 0);
    // partial S^T tiles over this wave's dims: rows 16 * rt + 4 * g + e, head r16
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (computes) {
      const uint32_t sb0 = bufa + sc_off0, sb1 = bufa + sc_off1;
      i32x4 sa[2][2 * SB];
      auto s_issue = [&](auto KB, i32x4(&a)[2 * SB]) {
        static_for<0, SB>([&](auto J) {
          constexpr int st = decltype(KB)::value * SB + decltype(J)::value;
          constexpr int off = 128 * (st >> 1);
          const uint32_t bse = (st & 1) ? sb1 : sb0;
          a[2 * J] = ds_read_b128_off<off>(bse);
          a[2 * J + 1] = ds_read_b128_off<off + 16 * ROWB>(bse);
        });
      };
      s_issue(std::integral_constant<int, 0>(), sa[0]);
      static_for<0, KSW / SB>([&](auto KB) {
        constexpr int kb = decltype(KB)::value;
        constexpr int cur = kb & 1;
        if constexpr (SB == 3)
          lds_wait6(sa[cur][0], sa[cur][1], sa[cur][2], sa[cur][3], sa[cur][4], sa[cur][5]);
        else
          lds_wait4(sa[cur][0], sa[cur][1], sa[cur][2], sa[cur][3]);
        if constexpr (kb + 1 < KSW / SB) s_issue(std::integral_constant<int, kb + 1>(), sa[cur ^ 1]);
        static_for<0, SB>([&](auto J) {
          sacc[0] = mma_bf16(sa[cur][2 * J], qreg[SB * kb + J], sacc[0]);
          sacc[1] = mma_bf16(sa[cur][2 * J + 1], qreg[SB * kb + J], sacc[1]);
        });
      });
      s_xch[wave][0][lane] = sacc[0];
      s_xch[wave][1][lane] = sacc[1];
    }
    lds_write_barrier();  // partial scores of both waves of a pair are in LDS
    if (computes) {
      const f32x4 p0 = s_xch[wave ^ 4][0][lane], p1 = s_xch[wave ^ 4][1][lane];
      // both waves of the pair add the halves in the same order, so they hold equal scores
      const f32x4 a0 = hf == 0 ? sacc[0] : p0, b0 = hf == 0 ? p0 : sacc[0];
      const f32x4 a1 = hf == 0 ? sacc[1] : p1, b1 = hf == 0 ? p1 : sacc[1];
      const uint32_t vlo = vbits >> (4 * g), vhi = vbits >> (16 + 4 * g);
      float z[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[e] = (vlo >> e) & 1u ? (a0[e] + b0[e]) * sm_scale : -INFINITY;
        z[4 + e] = (vhi >> e) & 1u ? (a1[e] + b1[e]) * sm_scale : -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      // m_run is a reference max, not the exact running max: weights are exp(z - m_run) and
      // O, l are kept relative to it. It moves (and O, l are rescaled) only when a tile's max
      // exceeds it by more than kLazyRescale, so weights stay below e^kLazyRescale (harmless
      // in fp32 and for the bf16 hi + lo split) and the rescale branch is rarely taken. O / l
      // and m_run + log(l) do not depend on the reference.
      // Every head sees the same valid rows, so mt is -inf in all lanes or in none.
      if (mt != -INFINITY) {
        if (__ballot(mt > m_run + kLazyRescale) != 0) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            o[t][0] *= alpha;
            o[t][1] *= alpha;
            o[t][2] *= alpha;
            o[t][3] *= alpha;
          }
          l_run *= alpha;
          m_run = m_new;
        }
        // p = hi + lo with both parts bf16 (hardware round to nearest even): the value
        // product runs once per part, so the weights keep about 16 significant bits.
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __expf(z[e] - m_run);  // exp(-inf) = 0
        bf16x8 hi8, lo8;
#pragma unroll
        for (int e = 0; e < 8; ++e) hi8[e] = (__bf16)p[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo8[e] = (__bf16)(p[e] - (float)hi8[e]);
        float psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        psum += shfl_xor(psum, 16);
        psum += shfl_xor(psum, 32);
        l_run += psum;
        // P^T operand: k slots 0..3 = rows 4g+e, slots 4..7 = rows 16+4g+e
        const i32x4 pv_hi = __builtin_bit_cast(i32x4, hi8);
        const i32x4 pv_lo = __builtin_bit_cast(i32x4, lo8);
        // V^T operand through transpose reads of this wave's output dims: lane i of row-group
        // g supplies the address of rows (4g + i/4) and (16 + 4g + i/4), dims 16T + 4*(i%4).
        // Batches of four output tiles; batch k+1 is in flight during batch k.
        uint32_t tb_[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) tb_[j] = bufa + tr_off[j];
        i16x4 lo[2][4], hi[2][4];
        auto tr_issue = [&](auto TB, i16x4(&l)[4], i16x4(&h)[4]) {
          static_for<0, 4>([&](auto J) {
            constexpr int off = 128 * decltype(TB)::value;
            l[J] = ds_read_tr16_off<off>(tb_[J]);
            h[J] = ds_read_tr16_off<off + 16 * ROWB>(tb_[J]);
          });
        };
        auto tr_wait = [&](i16x4(&l)[4], i16x4(&h)[4]) {
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(l[0]), "+v"(l[1]), "+v"(l[2]), "+v"(l[3]), "+v"(h[0]), "+v"(h[1]), "+v"(h[2]),
                         "+v"(h[3])
                       :
                       : "memory");
        };
        tr_issue(std::integral_constant<int, 0>(), lo[0], hi[0]);
        static_for<0, NTW / 4>([&](auto TB) {
          constexpr int tb = decltype(TB)::value;
          constexpr int cur = tb & 1;
          tr_wait(lo[cur], hi[cur]);
          if constexpr (tb + 1 < NTW / 4) tr_issue(std::integral_constant<int, tb + 1>(), lo[cur ^ 1], hi[cur ^ 1]);
          static_for<0, 4>([&](auto J) {
            constexpr int t = tb * 4 + decltype(J)::value;
            const i32x4 av = __builtin_bit_cast(i32x4, __builtin_shufflevector(lo[cur][J], hi[cur][J], 0, 1, 2, 3, 4, 5, 6, 7));
            o[t] = mma_bf16(av, pv_lo, mma_bf16(av, pv_hi, o[t]));
          });
        });
      }
    }
  }

  if (!computes) return;
  // lane holds O[head][256 * hf + 16t + 4g + e]
  const long qh = (long)bi * Hm + head;
  if (n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = out + qh * DL + 256 * hf + 4 * g;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      f32x4 v = o[t];
      v[0] *= inv;
      v[1] *= inv;
      v[2] *= inv;
      v[3] *= inv;
      *reinterpret_cast<f32x4*>(op + 16 * t) = v;
    }
    if (lse && hf == 0 && g == 0) lse[qh] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  } else {
    const long ph = ((long)bi * n_split + sp) * Hm + head;
    float* op = ws_o + ph * DL + 256 * hf + 4 * g;
#pragma unroll
    for (int t = 0; t < NTW; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = o[t];
    if (hf == 0 && g == 0) {
      ws_ml[2 * ph] = m_run;
      ws_ml[2 * ph + 1] = l_run;
    }
  }
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
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;  // over (query, head, dims / VEC)
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

int mla_auto_splits(int B, int n_q, int top_k) {
  const long rows = (long)B * n_q;
  long s = (256 + rows - 1) / rows;             // about one workgroup per CU
  long max_s = top_k / 128;                     // at least 128 slots per part
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
  const size_t parts = (size_t)B * n_q * n_split * Hm;
  return align256(parts * d_latent * sizeof(float)) + align256(parts * 2 * sizeof(float));
}

bool mla_mfma_supported(int Hm, int d_latent, int d_rope, int dtype) {
  return dtype == kBF16 && Hm % 16 == 0 && Hm <= 64 && d_latent == 512 && (d_rope == 64 || d_rope == 0);
}

hipError_t launch_sparse_mla(const void* q_abs, const void* latent, const int* idx,
                             const int* kv_len, float* out, float* lse, int B, int n_q, int Hm,
                             int n_kv, int top_k, int d_latent, int d_rope, float sm_scale,
                             int dtype, int n_split, void* workspace, hipStream_t stream) {
  const int chunk = (top_k + n_split - 1) / n_split;
  const long rows = (long)B * n_q;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (n_split > 1) {
    const size_t parts = (size_t)rows * n_split * Hm;
    ws_o = reinterpret_cast<float*>(workspace);
    ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                     align256(parts * d_latent * sizeof(float)));
  }
  if (mla_mfma_supported(Hm, d_latent, d_rope, dtype)) {
    const unsigned blocks = (unsigned)(rows * n_split);
    if (d_rope == 64)
      hipLaunchKernelGGL(sparse_mla_mfma<64>, dim3(blocks), dim3(512), 0, stream, (const bf16_t*)q_abs,
                         (const bf16_t*)latent, idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hm, n_kv,
                         top_k, sm_scale, n_split, chunk);
    else
      hipLaunchKernelGGL(sparse_mla_mfma<0>, dim3(blocks), dim3(512), 0, stream, (const bf16_t*)q_abs,
                         (const bf16_t*)latent, idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hm, n_kv,
                         top_k, sm_scale, n_split, chunk);
  } else {
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
  if (d_latent % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
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
