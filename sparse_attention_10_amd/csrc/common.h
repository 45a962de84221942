// Shared device helpers for the libdsa HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// 16-bit storage types: raw bits, decoded on the fly.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
  return (float)h;
}
// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> __device__ __forceinline__ float load_as_f32(const T* p, long i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float* p, long i) { return p[i]; }
template <> __device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p, long i) {
  return bf16_bits_to_f32(p[i].bits);
}
template <> __device__ __forceinline__ float load_as_f32<f16_t>(const f16_t* p, long i) {
  return f16_bits_to_f32(p[i].bits);
}

// Scores as order-preserving uint32 keys for selection: a larger score gives a larger key;
// -0.0 maps like +0.0; NaN and -inf map to 0, which marks "not a valid entry".
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (!(f == f)) return 0u;          // NaN
  if (u == 0xff800000u) return 0u;   // -inf
  if (u == 0x80000000u) u = 0u;      // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Cross-lane helpers (wave64). xor 16 / 32 move data between the four 16-lane rows.
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Workgroup -> XCD placement. The hardware deals consecutive workgroup ids round-robin
// over the 8 XCDs; remapping gives each XCD a contiguous range of logical ids so that
// neighbouring logical work items (which share inputs) share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  int per = total / kXcd;            // full rounds
  int full = per * kXcd;
  if (pid >= full) return pid;       // the ragged tail keeps its id
  int xcd = pid % kXcd;
  int slot = pid / kXcd;
  return xcd * per + slot;
}

}  // namespace dsa
