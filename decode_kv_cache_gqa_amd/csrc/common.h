// Device-side helpers shared by the library's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvev {

constexpr int kWave = 64;
constexpr int kPageTokens = 16;  // tokens per cache page

// bf16 is stored as its upper 16 bits of an IEEE binary32.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte vector of elements of T, widened to fp32.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const uint4& r, float* f) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// K pages are token-major: element (layer l, page p, row r, channel c) of a
// pool laid out [L][P][16][D] is at kidx(...).  V pages are channel-major,
// [L][P][D][16], so that 8 consecutive tokens of one channel are 16
// contiguous bytes: the operand layout of the p.V matrix-core product.
__device__ __forceinline__ int64_t kidx(int l, int page, int r, int c, int64_t P, int D) {
  return ((static_cast<int64_t>(l) * P + page) * kPageTokens + r) * D + c;
}
__device__ __forceinline__ int64_t vidx(int l, int page, int r, int c, int64_t P, int D) {
  return ((static_cast<int64_t>(l) * P + page) * D + c) * kPageTokens + r;
}

// Butterfly over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0x128>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x122>(v));
  return fmaxf(v, dpp_f<0x121>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  return v + dpp_f<0x121>(v);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace kvev
