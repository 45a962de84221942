// Indexer inputs of newly appended tokens, before scoring (ik_llama_opt commit log):
//   sub-commit "Add GLM-5.2/DeepSeek-V3.2 DSA lightning indexer": the indexer query (per head)
//   and key (one head) are split into a 64-dim rope part and a 64-dim nope part, the rope
//   part gets NeoX rotary embedding, and the parts are concatenated again;
//   sub-commit "decode-correct via persistent indexer-K cache": q and k are Hadamard-rotated
//   (orthonormal, so scores do not change) and the batch's keys are written into the
//   persistent key cache at their positions. The new 576-wide latent rows go into the MLA
//   cache the same way.
//
// NeoX rope pairs dim i with dim i + 32 (i < 32) and turns the pair by
// theta_i = pos * base^(-i/32). The rotation is Sylvester's 128-point Walsh-Hadamard matrix
// over sqrt(128), applied as a butterfly (x_j, x_{j+h}) -> (x_j + x_{j+h}, x_j - x_{j+h}) for
// h = 1, 2, ..., 64.
//
// Layout: 16 threads per 128-dim row, thread t holding dims 8t .. 8t+7 (two 16-byte loads of
// fp32 input, one 16-byte store of 16-bit output). The rope partner of dim i sits in thread
// t ^ 4; the butterflies with h >= 8 exchange with thread t ^ (h / 8). All exchanges stay
// inside the row's 16 lanes.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dsa {

constexpr int kPrepThreads = 256;  // 16 rows of 128 dims per workgroup

// base^(-i/32) / (2 pi) for the 32 rope pairs, in double (passed by value with the launch)
struct RopeTurns {
  double turns[32];
};

__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// 8 consecutive values to dst (out_dtype: F32 two 16-byte stores, else one)
__device__ __forceinline__ void store8(uint8_t* dst, const float (&v)[8], int out_dtype) {
  if (out_dtype == kF32) {
    reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else if (out_dtype == kBF16) {
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
  } else {
    *reinterpret_cast<uint4*>(dst) =
        make_uint4(pack2_f16(v[0], v[1]), pack2_f16(v[2], v[3]), pack2_f16(v[4], v[5]), pack2_f16(v[6], v[7]));
  }
}

// Rows [0, q_rows) are query rows (token r / H, head r % H); rows [q_rows, q_rows + k_rows)
// are key rows (token r - q_rows). pos[token] is the token's position and cache row.
__global__ __launch_bounds__(kPrepThreads) void indexer_prep_rows(
    const float* __restrict__ q_in, const float* __restrict__ k_in, const int* __restrict__ pos,
    uint8_t* __restrict__ q_out, uint8_t* __restrict__ k_cache, int q_rows, int k_rows, int H,
    int n_new, int n_kv, int out_dtype, RopeTurns freq, int hadamard) {
  const int t = threadIdx.x & 15;
  const long r = (long)blockIdx.x * (kPrepThreads / 16) + (threadIdx.x >> 4);
  if (r >= (long)q_rows + k_rows) return;  // whole 16-lane groups leave together
  const bool is_q = r < q_rows;
  const long token = is_q ? r / H : r - q_rows;
  const float* src = (is_q ? q_in + r * 128 : k_in + token * 128) + 8 * t;
  const int p = pos[token];

  float x[8];
  {
    const float4 a = reinterpret_cast<const float4*>(src)[0];
    const float4 b = reinterpret_cast<const float4*>(src)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }

  // NeoX rope on dims 0..63. The angle in turns, p * base^(-i/32) / (2 pi), is formed in double
  // and its fractional part taken there (positions reach 2^17 and more, where a float angle
  // would be off by 1e-2 rad); cos / sin then run in float on an angle in [-pi, pi].
  {
    float c[8], s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = 8 * (t & 3) + j;  // pair index i of dims (i, i + 32)
      const double turns = (double)p * freq.turns[f];
      const float red = (float)((turns - rint(turns)) * 6.283185307179586476925287);
      sincosf(red, &s[j], &c[j]);
    }
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float partner = __shfl_xor(x[j], 4, 64);
      if (t < 4) y[j] = x[j] * c[j] - partner * s[j];
      else if (t < 8) y[j] = x[j] * c[j] + partner * s[j];
      else y[j] = x[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = y[j];
  }

  if (hadamard) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j & h) == 0) {
          const float a = x[j], b = x[j + h];
          x[j] = a + b;
          x[j + h] = a - b;
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = __shfl_xor(x[j], m, 64);
        x[j] = (t & m) ? o - x[j] : x[j] + o;
      }
    const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= scale;
  }

  const int esz = out_dtype == kF32 ? 4 : 2;
  if (is_q) {
    store8(q_out + (r * 128 + 8 * t) * esz, x, out_dtype);
  } else if (p >= 0 && p < n_kv) {
    const long b = token / n_new;
    store8(k_cache + (((long)b * n_kv + p) * 128 + 8 * t) * esz, x, out_dtype);
  }
}

// latent rows: thread per 16-byte chunk; row_chunks chunks per row
__global__ __launch_bounds__(256) void cache_append_rows(const uint4* __restrict__ rows, const int* __restrict__ pos,
                                                         uint4* __restrict__ cache, long n_tok, int n_new, int n_kv,
                                                         int row_chunks) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_tok * row_chunks) return;
  const long token = e / row_chunks;
  const int c = (int)(e - token * row_chunks);
  const int p = pos[token];
  if (p < 0 || p >= n_kv) return;
  const long b = token / n_new;
  cache[((long)b * n_kv + p) * row_chunks + c] = rows[token * row_chunks + c];
}

hipError_t launch_indexer_prep(const float* q_in, const float* k_in, const void* latent_in, const int* pos,
                               void* q_out, void* k_cache, void* latent_cache, int B, int n_new, int H,
                               int n_kv, int row_bytes, int out_dtype, double log2_base, int hadamard,
                               hipStream_t stream) {
  RopeTurns freq;
  for (int i = 0; i < 32; ++i) freq.turns[i] = exp2(-(double)i / 32.0 * log2_base) / 6.283185307179586476925287;
  const long n_tok = (long)B * n_new;
  const long q_rows = q_in ? n_tok * H : 0;
  const long k_rows = k_in ? n_tok : 0;
  if (q_rows + k_rows > 0) {
    const long blocks = (q_rows + k_rows + 15) / 16;
    hipLaunchKernelGGL(indexer_prep_rows, dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream, q_in, k_in, pos,
                       (uint8_t*)q_out, (uint8_t*)k_cache, (int)q_rows, (int)k_rows, H, n_new, n_kv, out_dtype,
                       freq, hadamard);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (latent_in) {
    const int row_chunks = row_bytes / 16;
    const long total = n_tok * row_chunks;
    hipLaunchKernelGGL(cache_append_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       (const uint4*)latent_in, pos, (uint4*)latent_cache, n_tok, n_new, n_kv, row_chunks);
  }
  return hipGetLastError();
}

}  // namespace dsa
