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
// Layout: 8 threads per 128-dim row, thread t holding dims 16t .. 16t+15 (four 16-byte loads of
// fp32 input, two 16-byte stores of 16-bit output). The rope partner of dim i sits in thread
// t ^ 2; the butterflies with h <= 8 stay in the thread, those with h = 16, 32, 64 exchange
// with thread t ^ 1, t ^ 2, t ^ 4. All exchanges are DPP lane moves inside the row's 8 lanes
// (quad permutes for ^1 and ^2, a row shift either way for ^4), so no LDS traffic is involved.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace dsa {

constexpr int kPrepThreads = 256;  // 32 rows of 128 dims per workgroup
constexpr int kPrepTpr = 8;        // threads per row

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
__device__ __forceinline__ void store8(uint8_t* dst, const float* v, int out_dtype) {
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

// DPP lane moves within 4-lane quads (lane ^ 1, lane ^ 2) and 8-lane groups (lane ^ 4)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_xor1(float x) { return dpp<0xB1>(x); }  // quad_perm [1,0,3,2]
__device__ __forceinline__ float lane_xor2(float x) { return dpp<0x4E>(x); }  // quad_perm [2,3,0,1]
__device__ __forceinline__ float lane_xor4(float x, bool hi) {
  const float up = dpp<0x104>(x);    // row_shl:4, the value of lane + 4
  const float down = dpp<0x114>(x);  // row_shr:4, the value of lane - 4
  return hi ? down : up;
}

// Workgroup (token, chunk): rows 32 * chunk .. + 31 of the token's rows, which are its nq
// query heads followed by its key (nk = 0 or 1). The rope angles depend on the token only, so
// 32 threads compute the 32 (cos, sin) pairs once into LDS for all the token's rows.
__global__ __launch_bounds__(kPrepThreads) void indexer_prep_rows(
    const float* __restrict__ q_in, const float* __restrict__ k_in, const int* __restrict__ pos,
    uint8_t* __restrict__ q_out, uint8_t* __restrict__ k_cache, int nq, int nk, int n_new, int n_kv,
    int out_dtype, RopeTurns freq, int hadamard) {
  __shared__ float s_cos[32], s_sin[32];
  const int t = threadIdx.x & (kPrepTpr - 1);
  const long token = blockIdx.x;
  const int p = pos[token];
  if (threadIdx.x < 32) {
    // the angle in turns, p * base^(-i/32) / (2 pi), is formed in double and its fractional
    // part taken there (positions reach 2^17 and more, where a float angle would be off by
    // 1e-2 rad); cos / sin then run in float on an angle in [-pi, pi]
    const double turns = (double)p * freq.turns[threadIdx.x];
    const float red = (float)((turns - rint(turns)) * 6.283185307179586476925287);
    float sn, cs;
    sincosf(red, &sn, &cs);
    s_cos[threadIdx.x] = cs;
    s_sin[threadIdx.x] = sn;
  }
  __syncthreads();
  const int j_row = blockIdx.y * (kPrepThreads / kPrepTpr) + (int)(threadIdx.x / kPrepTpr);
  // Rows past the token's last compute on its first row and store nothing: every lane of a
  // row group stays active for the lane moves.
  const bool live = j_row < nq + nk;
  const int jr = live ? j_row : 0;
  const bool is_q = jr < nq;
  const float* src = (is_q ? q_in + (token * nq + jr) * 128 : k_in + token * 128) + 16 * t;

  float x[16];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = reinterpret_cast<const float4*>(src)[c];
    x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
  }

  // NeoX rope on dims 0..63 (threads 0..3; thread t pairs with t ^ 2)
  {
    const bool rope = t < 4;
    const bool upper = (t & 2) != 0;  // holds dims i + 32
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float partner = lane_xor2(x[j]);
      const int f = 16 * (t & 1) + j;
      const float c = s_cos[f], sn = s_sin[f];
      const float y = upper ? x[j] * c + partner * sn : x[j] * c - partner * sn;
      x[j] = rope ? y : x[j];
    }
  }

  if (hadamard) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((j & h) == 0) {
          const float a = x[j], b = x[j + h];
          x[j] = a + b;
          x[j + h] = a - b;
        }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float o = lane_xor1(x[j]);
      x[j] = (t & 1) ? o - x[j] : x[j] + o;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float o = lane_xor2(x[j]);
      x[j] = (t & 2) ? o - x[j] : x[j] + o;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float o = lane_xor4(x[j], (t & 4) != 0);
      x[j] = (t & 4) ? o - x[j] : x[j] + o;
    }
    const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] *= scale;
  }

  if (!live) return;
  const int esz = out_dtype == kF32 ? 4 : 2;
  uint8_t* dst = nullptr;
  if (is_q) {
    dst = q_out + ((token * nq + jr) * 128 + 16 * t) * esz;
  } else if (p >= 0 && p < n_kv) {
    const long b = token / n_new;
    dst = k_cache + (((long)b * n_kv + p) * 128 + 16 * t) * esz;
  }
  if (dst) {
    store8(dst, x, out_dtype);
    store8(dst + 8 * esz, x + 8, out_dtype);
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
  const int nq = q_in ? H : 0, nk = k_in ? 1 : 0;
  if (nq + nk > 0) {
    const int rows_per_block = kPrepThreads / kPrepTpr;
    dim3 grid((unsigned)n_tok, (unsigned)((nq + nk + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL(indexer_prep_rows, grid, dim3(kPrepThreads), 0, stream, q_in, k_in, pos, (uint8_t*)q_out,
                       (uint8_t*)k_cache, nq, nk, n_new, n_kv, out_dtype, freq, hadamard);
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
