// Pooled indexer (vllm-rdna pull request "Glm5Next (GLM-5.3-Flash) on gfx1030": architecture
// section and the DSA attention and first-cut kernel commits). The indexer cache holds one
// packed row per token, k[D] | gate[D] | valid; groups of kpool = 4 consecutive tokens are
// compressed into one pool key with softmax(gate + ape) weights; queries score pool keys with
// the ordinary indexer score; top-k keeps top_k / kpool pools; the attended tokens are the
// selected pools' tokens plus the last incomplete pool (the tail, at most kpool - 1 tokens),
// which is always attended: 2048 + 3 = 2051 for top_k 2048.
//
//   kpool_compress: key[p][d] = sum_j softmax_j(gate[t_j][d] + ape[j][d]) k[t_j][d], the sum
//     over the pool's valid tokens t_j = kpool p + j; a pool without valid tokens is zero.
//     One thread per (pool, dim): consecutive threads read consecutive 16-bit values of the
//     pool's rows, which lie back to back in the cache.
//   kpool_expand: one thread per output slot; selected pools first (kpool tokens each, in
//     pool order), then the tail tokens kpool floor((pos + 1) / kpool) .. pos; -1 for padding,
//     tokens whose valid entry is zero and tokens outside the cache.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dsa {

constexpr int kMaxPool = 8;

template <typename T>
__device__ __forceinline__ bool valid_entry(const T* row, int col);
template <>
__device__ __forceinline__ bool valid_entry<float>(const float* row, int col) {
  return (__float_as_uint(row[col]) & 0x7fffffffu) != 0u;
}
template <>
__device__ __forceinline__ bool valid_entry<bf16_t>(const bf16_t* row, int col) {
  return (row[col].bits & 0x7fffu) != 0u;
}
template <>
__device__ __forceinline__ bool valid_entry<f16_t>(const f16_t* row, int col) {
  return (row[col].bits & 0x7fffu) != 0u;
}

template <typename T>
__device__ __forceinline__ void store_as(T* p, long i, float v);
template <>
__device__ __forceinline__ void store_as<float>(float* p, long i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store_as<bf16_t>(bf16_t* p, long i, float v) {
  p[i].bits = (uint16_t)f32_to_bf16_bits(v);
}
template <>
__device__ __forceinline__ void store_as<f16_t>(f16_t* p, long i, float v) {
  p[i].bits = __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}

// grid (ceil(n_pools * D / 256), B); pools [p0, p0 + n_pools) of every sequence
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void kpool_compress(const TI* __restrict__ packed, long stride,
                                                      const float* __restrict__ ape, TO* __restrict__ pooled,
                                                      int n_kv, int D, int kpool, int p0, int n_pools) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long)n_pools * D) return;
  const int b = blockIdx.y;
  const int p = p0 + (int)(e / D);
  const int d = (int)(e - (long)(p - p0) * D);
  const TI* rows = packed + ((long)b * n_kv + (long)kpool * p) * stride;
  float a[kMaxPool], kv[kMaxPool];
  bool ok[kMaxPool];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxPool; ++j) {
    ok[j] = false;
    a[j] = 0.f;
    kv[j] = 0.f;
    if (j < kpool) {
      const TI* row = rows + (long)j * stride;
      ok[j] = valid_entry(row, 2 * D);
      a[j] = load_as_f32(row, D + d) + ape[j * D + d];
      kv[j] = load_as_f32(row, d);
      if (ok[j]) m = fmaxf(m, a[j]);
    }
  }
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPool; ++j)
    if (ok[j]) {
      const float x = expf(a[j] - m);
      den += x;
      num = fmaf(x, kv[j], num);
    }
  const int n_pool_cap = n_kv / kpool;
  store_as(pooled, ((long)b * n_pool_cap + p) * D + d, den > 0.f ? num / den : 0.f);
}

// grid (ceil(width / 256), B * n_q)
template <typename TI>
__global__ __launch_bounds__(256) void kpool_expand(const int* __restrict__ pool_idx, const TI* __restrict__ packed,
                                                    long stride, int D, const int* __restrict__ kv_len,
                                                    const int* __restrict__ q_pos, int* __restrict__ tok_idx,
                                                    int n_q, int n_kv, int top_pools, int kpool) {
  const int width = kpool * top_pools + kpool - 1;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= width) return;
  const long bi = blockIdx.y;
  const int b = (int)(bi / n_q), i = (int)(bi - (long)b * n_q);
  const long len = kv_len ? min((long)kv_len[b], (long)n_kv) : (long)n_kv;
  long t;
  if (s < kpool * top_pools) {
    const int p = pool_idx[bi * top_pools + s / kpool];
    t = p < 0 ? -1 : (long)kpool * p + s % kpool;
  } else {
    const long pos = q_pos ? (long)q_pos[bi] : len - n_q + i;
    const long first = pos + 1 >= 0 ? (pos + 1) / kpool * kpool : -1;  // tail start
    t = first < 0 ? -1 : first + (s - kpool * top_pools);
    if (t > pos) t = -1;
  }
  int out = -1;
  if (t >= 0 && t < len && valid_entry(packed + ((long)b * n_kv + t) * stride, 2 * D)) out = (int)t;
  tok_idx[bi * width + s] = out;
}

template <typename TI>
static hipError_t compress_to(const void* packed, long stride, const float* ape, void* pooled, int out_dtype,
                              int B, int n_kv, int D, int kpool, int p0, int n_pools, hipStream_t stream) {
  const dim3 grid((unsigned)(((long)n_pools * D + 255) / 256), (unsigned)B);
  const TI* in = (const TI*)packed;
  if (out_dtype == kF32)
    hipLaunchKernelGGL((kpool_compress<TI, float>), grid, dim3(256), 0, stream, in, stride, ape, (float*)pooled,
                       n_kv, D, kpool, p0, n_pools);
  else if (out_dtype == kBF16)
    hipLaunchKernelGGL((kpool_compress<TI, bf16_t>), grid, dim3(256), 0, stream, in, stride, ape,
                       (bf16_t*)pooled, n_kv, D, kpool, p0, n_pools);
  else
    hipLaunchKernelGGL((kpool_compress<TI, f16_t>), grid, dim3(256), 0, stream, in, stride, ape, (f16_t*)pooled,
                       n_kv, D, kpool, p0, n_pools);
  return hipGetLastError();
}

hipError_t launch_kpool_compress(const void* packed, int row_stride, int row_dtype, const float* ape,
                                 void* pooled, int out_dtype, int B, int n_kv, int D, int kpool,
                                 int pool_begin, int pool_end, hipStream_t stream) {
  const int n_pools = pool_end - pool_begin;
  if (n_pools <= 0) return hipSuccess;
  if (row_dtype == kF32)
    return compress_to<float>(packed, row_stride, ape, pooled, out_dtype, B, n_kv, D, kpool, pool_begin, n_pools,
                              stream);
  if (row_dtype == kBF16)
    return compress_to<bf16_t>(packed, row_stride, ape, pooled, out_dtype, B, n_kv, D, kpool, pool_begin,
                               n_pools, stream);
  return compress_to<f16_t>(packed, row_stride, ape, pooled, out_dtype, B, n_kv, D, kpool, pool_begin, n_pools,
                            stream);
}

hipError_t launch_kpool_expand(const int* pool_idx, const void* packed, int row_stride, int row_dtype, int D,
                               const int* kv_len, const int* q_pos, int* tok_idx, int B, int n_q, int n_kv,
                               int top_pools, int kpool, hipStream_t stream) {
  const int width = kpool * top_pools + kpool - 1;
  const dim3 grid((unsigned)((width + 255) / 256), (unsigned)((long)B * n_q));
  if (row_dtype == kF32)
    hipLaunchKernelGGL(kpool_expand<float>, grid, dim3(256), 0, stream, pool_idx, (const float*)packed,
                       (long)row_stride, D, kv_len, q_pos, tok_idx, n_q, n_kv, top_pools, kpool);
  else if (row_dtype == kBF16)
    hipLaunchKernelGGL(kpool_expand<bf16_t>, grid, dim3(256), 0, stream, pool_idx, (const bf16_t*)packed,
                       (long)row_stride, D, kv_len, q_pos, tok_idx, n_q, n_kv, top_pools, kpool);
  else
    hipLaunchKernelGGL(kpool_expand<f16_t>, grid, dim3(256), 0, stream, pool_idx, (const f16_t*)packed,
                       (long)row_stride, D, kv_len, q_pos, tok_idx, n_q, n_kv, top_pools, kpool);
  return hipGetLastError();
}

}  // namespace dsa
