// Device helpers shared by the gfx950 kernels: bf16 conversion, RoPE angles,
// wave64 cross-lane sums, order-preserving float keys, block scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest, ties to even (inputs are finite).
// float -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// float -> FP8 E5M2 byte (1 sign, 5 exponent bits with bias 15, 2 mantissa bits),
// round to nearest, ties to even; below 2^-14 the values are multiples of 2^-16;
// magnitudes that round past 57344 give inf.  Inputs are finite.
__device__ __forceinline__ uint8_t f32_to_e5m2(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float x = fabsf(f);
  if (x < 0x1p-14f) return (uint8_t)(sign | (uint32_t)rintf(x * 65536.0f));   // 4 -> smallest normal
  uint32_t v = __float_as_uint(x);
  v += 0xfffffu + ((v >> 21) & 1u);              // round the 21 dropped mantissa bits
  const int e = (int)(v >> 23) - 127 + 15;
  if (e >= 31) return (uint8_t)(sign | 0x7cu);   // inf
  return (uint8_t)(sign | ((uint32_t)e << 2) | ((v >> 21) & 3u));
}

// double -> bf16 bits, one rounding to nearest even at the 8th significant bit
// (the double is cut to 8 significant bits first, which float holds exactly).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u += (1ull << 44) - 1ull + ((u >> 45) & 1ull);
  u &= ~((1ull << 45) - 1ull);
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

// double -> FP8 E5M2 byte, one rounding to nearest even (2 mantissa bits kept;
// below 2^-14 the grid is 2^-16; past 57344 the result is inf).
__device__ __forceinline__ uint8_t f64_to_e5m2_rne(double x) {
  const uint32_t sign = (uint32_t)((uint64_t)__double_as_longlong(x) >> 56) & 0x80u;
  const double ax = fabs(x);
  if (ax < 0x1p-14) return (uint8_t)(sign | (uint32_t)rint(ax * 65536.0));
  uint64_t v = (uint64_t)__double_as_longlong(ax);
  v += (1ull << 49) - 1ull + ((v >> 50) & 1ull);
  const int e = (int)(v >> 52) - 1023 + 15;
  if (e >= 31) return (uint8_t)(sign | 0x7cu);
  return (uint8_t)(sign | ((uint32_t)e << 2) | (uint32_t)((v >> 50) & 3ull));
}

// Unpack 8 bf16 held in a 16-byte word into floats.
__device__ __forceinline__ void unpack8(const u32x4 w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

// ---------------------------------------------------------------- RoPE

// cos/sin of pos * inv_freq entirely in float64: the product and the reduction
// modulo 2*pi (positions up to 2^20 lose nothing), then the float64 sincos of the
// reduced angle.  Used where a rotated key is
// rounded once to its storage format (landmarks, exact outlier / window keys,
// exact generated keys), so that the rounding sees the float64 value.
__device__ __forceinline__ void rope_cs64(int64_t pos, double inv_freq, double* c, double* s) {
  const double two_pi_hi = 6.283185307179586;
  const double two_pi_lo = 2.4492935982947064e-16;
  double a = (double)pos * inv_freq;
  double n = rint(a * 0.15915494309189535);
  double r = fma(-n, two_pi_hi, a);
  r = fma(-n, two_pi_lo, r);
  sincos(r, s, c);
}

// pos * inv_freq reduced to [-pi, pi] in float64, returned as float.
__device__ __forceinline__ float rope_angle(int64_t pos, double inv_freq) {
  const double two_pi_hi = 6.283185307179586;
  const double two_pi_lo = 2.4492935982947064e-16;
  double a = (double)pos * inv_freq;
  double n = rint(a * 0.15915494309189535);
  double r = fma(-n, two_pi_hi, a);
  return (float)fma(-n, two_pi_lo, r);
}

// ---------------------------------------------------------------- cross-lane

// DPP controls (gfx9 encoding).
#define SKV_DPP_QP_XOR1 0xB1     // quad_perm [1,0,3,2]
#define SKV_DPP_QP_XOR2 0x4E     // quad_perm [2,3,0,1]
#define SKV_DPP_ROW_HALF_MIRROR 0x141
#define SKV_DPP_ROW_MIRROR 0x140
#define SKV_DPP_ROW_SHR(n) (0x110 + (n))
#define SKV_DPP_ROW_BCAST15 0x142  // lane 15 of each row to the next row (gfx9)
#define SKV_DPP_ROW_BCAST31 0x143  // lane 31 to rows 2 and 3 (gfx9)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<SKV_DPP_QP_XOR1>(v);
  v += dpp<SKV_DPP_QP_XOR2>(v);
  v += dpp<SKV_DPP_ROW_HALF_MIRROR>(v);
  v += dpp<SKV_DPP_ROW_MIRROR>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Wave-uniform minimum / maximum of a uint32: DPP within each row of 16 lanes,
// then the four rows' results read as scalars (no LDS round trips).
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dppu<SKV_DPP_QP_XOR1>(v));
  v = min(v, dppu<SKV_DPP_QP_XOR2>(v));
  v = min(v, dppu<SKV_DPP_ROW_HALF_MIRROR>(v));
  v = min(v, dppu<SKV_DPP_ROW_MIRROR>(v));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dppu<SKV_DPP_QP_XOR1>(v));
  v = max(v, dppu<SKV_DPP_QP_XOR2>(v));
  v = max(v, dppu<SKV_DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dppu<SKV_DPP_ROW_MIRROR>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts by 1, 2, 4, 8
// (lanes shifted in from outside a row add 0), then lane 15 of rows 0 and 2
// into rows 1 and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_SHR(1), 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_SHR(2), 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_SHR(4), 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_SHR(8), 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_BCAST15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, SKV_DPP_ROW_BCAST31, 0xC, 0xF, false);
  return x;
}

// ---------------------------------------------------------------- keys

// Order-preserving map of a finite float to uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- block scan

// Exclusive prefix sum over a block of NT threads (NT multiple of 64, <= 1024).
// `tmp` needs NT/64 ints of LDS.  Returns the exclusive prefix, writes the total.
// TRAIL = false leaves out the closing barrier: the caller passes another barrier
// before anything writes tmp again.
template <int NT, bool TRAIL = true>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; w++) {
    int t = tmp[w];
    if (w < wid) base += t;
    tot += t;
  }
  if constexpr (TRAIL) __syncthreads();
  *total = tot;
  return base + x - v;
}

}  // namespace skv
