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
__device__ __forceinline__ i16x4 ds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <int DR>
__global__ __launch_bounds__(256) void sparse_mla_mfma(
    const bf16_t* __restrict__ qa, const bf16_t* __restrict__ lat, const int* __restrict__ idx,
    const int* __restrict__ kv_len, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_q, int Hm, int n_kv, int top_k,
    float sm_scale, int n_split, int chunk) {
  constexpr int DL = 512;
  constexpr int DC = DL + DR;
  constexpr int ROWB = DC * 2;              // bytes per row
  constexpr int RS = ROWB + 16;             // LDS row stride (padding breaks bank aliasing)
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int TILE_CHUNKS = kMlaRows * CPR;
  constexpr int CPT = (TILE_CHUNKS + 255) / 256;  // chunks per thread per tile
  constexpr int KS = DC / 32;               // k-steps of the score MFMA
  constexpr int NT = DL / 16;               // 16-dim output tiles

  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kMlaRows * RS];
  __shared__ int s_idx[kMlaMaxChunk];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bi = logical / n_split;
  const int sp = logical - bi * n_split;
  const int b = bi / n_q;
  const int len = kv_len ? min(kv_len[b], n_kv) : n_kv;
  const int s0 = sp * chunk, s1 = min(top_k, s0 + chunk);
  const int nslots = max(0, s1 - s0);
  const bool computes = wave * 16 < Hm;
  const int head = wave * 16 + r16;

  for (int j = tid; j < nslots; j += 256) {
    const int r = idx[(long)bi * top_k + s0 + j];
    s_idx[j] = (r >= 0 && r < len) ? r : -1;
  }

  // query operand (B of the score MFMA): lane holds head, dims 32*s + 8*g .. +8
  i32x4 qreg[KS];
  if (computes) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(qa) + ((long)bi * Hm + head) * ROWB;
#pragma unroll
    for (int s = 0; s < KS; ++s) qreg[s] = *reinterpret_cast<const i32x4*>(qp + (4 * s + g) * 16);
  }
  f32x4 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();

  const uint8_t* latb = reinterpret_cast<const uint8_t*>(lat) + (long)b * n_kv * ROWB;
  i32x4 pre[CPT];
  auto issue = [&](int tile) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + 256 * j;
      const int r = q / CPR, c = q - r * CPR;
      const int slot = tile * kMlaRows + r;
      pre[j] = i32x4{0, 0, 0, 0};
      if (q < TILE_CHUNKS && slot < nslots) {
        const int row = s_idx[slot];
        if (row >= 0) pre[j] = *reinterpret_cast<const i32x4*>(latb + (long)row * ROWB + c * 16);
      }
    }
  };
  auto stash = [&](uint8_t* buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int q = tid + 256 * j;
      const int r = q / CPR, c = q - r * CPR;
      if (q < TILE_CHUNKS) *reinterpret_cast<i32x4*>(buf + r * RS + c * 16) = pre[j];
    }
  };

  const int ntiles = (nslots + kMlaRows - 1) / kMlaRows;
  if (ntiles > 0) issue(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    uint8_t* buf = s_tile[tile & 1];
    stash(buf);
    __syncthreads();
    if (tile + 1 < ntiles) issue(tile + 1);
    if (computes) {
      // S^T tiles: rows 16*rt + 4*g + e, head r16
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const i32x4 a = *reinterpret_cast<const i32x4*>(buf + (16 * rt + r16) * RS + (4 * s + g) * 16);
          sacc[rt] = mma_bf16(a, qreg[s], sacc[rt]);
        }
      }
      float z[8];
      float mt = -INFINITY;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int slot = tile * kMlaRows + 16 * rt + 4 * g + e;
          const bool valid = slot < nslots && s_idx[slot] >= 0;
          const float v = valid ? sacc[rt][e] * sm_scale : -INFINITY;
          z[rt * 4 + e] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      float alpha = 1.f;
      // p = hi + lo with both parts bf16: the value product runs twice, once per part, so
      // the weights keep about 16 significant bits instead of bf16's 8.
      uint32_t ph[8], pl[8];
      float psum = 0.f;
      if (m_new != -INFINITY) {
        alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = z[e] == -INFINITY ? 0.f : __expf(z[e] - m_new);
          ph[e] = f32_to_bf16_bits(p);
          pl[e] = f32_to_bf16_bits(p - bf16_bits_to_f32(ph[e]));
          psum += p;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ph[e] = pl[e] = 0u;
      }
      psum += shfl_xor(psum, 16);
      psum += shfl_xor(psum, 32);
      l_run = alpha * l_run + psum;
      m_run = m_new;
      // P^T operand: k slots 0..3 = rows 4g+e, slots 4..7 = rows 16+4g+e
      const i32x4 pv_hi = {(int)(ph[0] | (ph[1] << 16)), (int)(ph[2] | (ph[3] << 16)),
                           (int)(ph[4] | (ph[5] << 16)), (int)(ph[6] | (ph[7] << 16))};
      const i32x4 pv_lo = {(int)(pl[0] | (pl[1] << 16)), (int)(pl[2] | (pl[3] << 16)),
                           (int)(pl[4] | (pl[5] << 16)), (int)(pl[6] | (pl[7] << 16))};
      // V^T operand through transpose reads: lane i of row-group g supplies the address of
      // rows (4g + i/4) and (16 + 4g + i/4), dims 16t + 4*(i%4) .. +4
      const uint8_t* va = buf + (4 * g + (r16 >> 2)) * RS + (r16 & 3) * 8;
      const uint8_t* vb = va + 16 * RS;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const i16x4 lo = ds_read_tr16(va + t * 32);
        const i16x4 hi = ds_read_tr16(vb + t * 32);
        const i32x4 av = {(int)(((uint32_t)(uint16_t)lo[0]) | ((uint32_t)(uint16_t)lo[1] << 16)),
                          (int)(((uint32_t)(uint16_t)lo[2]) | ((uint32_t)(uint16_t)lo[3] << 16)),
                          (int)(((uint32_t)(uint16_t)hi[0]) | ((uint32_t)(uint16_t)hi[1] << 16)),
                          (int)(((uint32_t)(uint16_t)hi[2]) | ((uint32_t)(uint16_t)hi[3] << 16))};
        f32x4 acc = o[t];
        acc[0] *= alpha;
        acc[1] *= alpha;
        acc[2] *= alpha;
        acc[3] *= alpha;
        acc = mma_bf16(av, pv_hi, acc);
        o[t] = mma_bf16(av, pv_lo, acc);
      }
    }
    __syncthreads();
  }

  if (!computes) return;
  // lane holds O[head][16t + 4g + e]
  const long qh = (long)bi * Hm + head;
  if (n_split == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* op = out + qh * DL + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 v = o[t];
      v[0] *= inv;
      v[1] *= inv;
      v[2] *= inv;
      v[3] *= inv;
      *reinterpret_cast<f32x4*>(op + 16 * t) = v;
    }
    if (lse && g == 0) lse[qh] = l_run > 0.f ? m_run + __logf(l_run) : -INFINITY;
  } else {
    const long ph = ((long)bi * n_split + sp) * Hm + head;
    float* op = ws_o + ph * DL + 4 * g;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(op + 16 * t) = o[t];
    if (g == 0) {
      ws_ml[2 * ph] = m_run;
      ws_ml[2 * ph + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------------------
// merge: one block of 128 threads per (query, head)
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void mla_merge(const float* __restrict__ ws_o,
                                                 const float* __restrict__ ws_ml,
                                                 float* __restrict__ out, float* __restrict__ lse,
                                                 int Hm, int n_split, int d_latent) {
  const long qh = blockIdx.x;  // (b * n_q + i) * Hm + h
  const long bi = qh / Hm;
  const int h = (int)(qh - bi * Hm);
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, ws_ml[2 * ((bi * n_split + s) * Hm + h)]);
  float L = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const long ph = (bi * n_split + s) * Hm + h;
    const float m = ws_ml[2 * ph];
    if (m != -INFINITY) L += __expf(m - M) * ws_ml[2 * ph + 1];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = threadIdx.x; d < d_latent; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const long ph = (bi * n_split + s) * Hm + h;
      const float m = ws_ml[2 * ph];
      if (m != -INFINITY) acc = fmaf(__expf(m - M), ws_o[ph * d_latent + d], acc);
    }
    out[qh * d_latent + d] = acc * inv;
  }
  if (lse && threadIdx.x == 0) lse[qh] = L > 0.f ? M + __logf(L) : -INFINITY;
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
      hipLaunchKernelGGL(sparse_mla_mfma<64>, dim3(blocks), dim3(256), 0, stream, (const bf16_t*)q_abs,
                         (const bf16_t*)latent, idx, kv_len, out, lse, ws_o, ws_ml, n_q, Hm, n_kv,
                         top_k, sm_scale, n_split, chunk);
    else
      hipLaunchKernelGGL(sparse_mla_mfma<0>, dim3(blocks), dim3(256), 0, stream, (const bf16_t*)q_abs,
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
  hipLaunchKernelGGL(mla_merge, dim3((unsigned)(rows * Hm)), dim3(128), 0, stream, ws_o, ws_ml, out,
                     lse, Hm, n_split, d_latent);
  return hipGetLastError();
}

}  // namespace dsa
