// Shared device helpers of libmetis_fp4 (gfx950 only).
//
// Number formats follow the public format descriptions (the Metis pages name
// MXFP4 and NVFP4 but do not define them):
//   E2M1  -- OCP Microscaling Formats v1.0 §5.3.3: magnitudes 0,.5,1,1.5,2,3,4,6
//   E8M0  -- OCP MX v1.0 §5.4.1, shared-exponent rule of §6.3
//   E4M3  -- OCP 8-bit FP "E4M3FN": bias 7, max 448, no infinities
// Rounding is to nearest with ties to the even code, saturating.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "metis_fp4.h"

namespace metis {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short ushortx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, unsigned short &hi, unsigned short &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Load element i of a row of type T as fp32.
template <typename T> __device__ __forceinline__ float load_f32(const T *p);
template <> __device__ __forceinline__ float load_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_f32<unsigned short>(const unsigned short *p) {
  return bf16_to_f32(*p);
}

// ------------------------------------------------------------------ E2M1
// Code (sign in bit 3) of the E2M1 value nearest to v. The count of decision
// points passed gives the magnitude index; at a decision point the even index
// wins (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4,
// 5 -> 4); above 5 everything saturates to 6.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const float a = fabsf(v);
  uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}

// Eight E2M1 codes (element j in nibble j) by the gfx950 FP4 conversion at
// scale 1: round to nearest even, saturating at 6, a zero keeping its sign.
// These are exactly the codes of e2m1_rne (equal on every finite float).
__device__ __forceinline__ uint32_t e2m1_pack8(const float *v) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
}

// Codes of one block of B pre-scaled values, packed eight to a word.
template <int B>
__device__ __forceinline__ void e2m1_pack(const float (&q)[B], uint32_t (&packed)[B / 8]) {
#pragma unroll
  for (int w = 0; w < B / 8; ++w) packed[w] = e2m1_pack8(&q[8 * w]);
}

// The fp32 value 2^e for e in [-127, 127] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_f32(int e) {
  return e > -127 ? __uint_as_float((uint32_t)(e + 127) << 23) : __uint_as_float(0x00400000u);
}

// Codes of one block of B values divided by the power of two `scale`: the
// gfx950 FP4 conversion divides its inputs by its scale operand before
// rounding, which for a power of two is exact (subnormal scales included), so
// these are the codes of e2m1_rne(v / scale) without a separate scaling step.
template <int B>
__device__ __forceinline__ void e2m1_pack_scaled(const float (&v)[B], float scale, uint32_t (&packed)[B / 8]) {
#pragma unroll
  for (int w = 0; w < B / 8; ++w) {
    const float *x = &v[8 * w];
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[2], x[3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[4], x[5], scale, 2);
    packed[w] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[6], x[7], scale, 3);
  }
}

// Magnitude of an E2M1 code times 2 (integers 0,1,2,3,4,6,8,12): value = x2 / 2.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t m = code & 7u;
  // 0, .5, 1, 1.5 for m < 4; 2, 3, 4, 6 for m >= 4
  float mag = (m < 4u) ? 0.5f * (float)m : (float)(2u << ((m - 4u) >> 1)) * ((m & 1u) ? 1.5f : 1.0f);
  return (code & 8u) ? -mag : mag;
}

// ------------------------------------------------------------------ E8M0
// MXFP4 shared exponent of a block with max magnitude amax >= 0:
// floor(log2 amax) - 2 clamped to [-127, 127]; -127 (byte 0) for amax == 0.
__device__ __forceinline__ int mx_shared_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  const uint32_t b = __float_as_uint(amax);
  const int field = (int)((b >> 23) & 0xFFu);
  int e;
  if (field == 0) {
    e = (31 - __clz(b & 0x7FFFFFu)) - 149;  // subnormal: leading bit position
  } else {
    e = field - 127;
  }
  e -= 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------------------ E4M3
// Non-negative fp32 -> E4M3FN byte, nearest even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float b) {
  if (!(b > 0.0f)) return 0u;
  if (b >= 448.0f) return 0x7Eu;
  const uint32_t u = __float_as_uint(b);
  const int e = (int)((u >> 23) & 0xFFu) - 127;
  if (e < -6) {
    // subnormal E4M3 range: multiples of 2^-9 (rintf rounds half to even);
    // a result of 8 steps is 2^-6, whose byte 0x08 is the same integer
    return (uint32_t)rintf(ldexpf(b, 9));
  }
  uint32_t keep = (u >> 20) & 7u;  // top three mantissa bits
  const uint32_t rest = u & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep++;
  uint32_t field = (uint32_t)(e + 7);
  if (keep == 8u) {
    keep = 0u;
    field++;
  }
  if (field > 15u || (field == 15u && keep > 6u)) return 0x7Eu;
  return (field << 3) | keep;
}

__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  const uint32_t field = (byte >> 3) & 15u, mant = byte & 7u;
  return field == 0u ? ldexpf((float)mant, -9) : ldexpf((float)(8u + mant), (int)field - 10);
}

// NVFP4 tensor scale from the tensor's max magnitude (fp32 ops, division).
__device__ __forceinline__ float nv_tensor_scale(float amax_tensor) {
  if (!(amax_tensor > 0.0f)) return 1.0f;
  const float s = __fdiv_rn(amax_tensor, 2688.0f);
  return s < 1.17549435e-38f ? 1.17549435e-38f : s;
}

// ------------------------------------------------------------------ MFMA
// 16x16x32 bf16 -> fp32. Lane l supplies row (or column) l % 16 and the eight
// contraction slots 8*(l/16) .. +7; the result holds rows 4*(l/16) .. +3 of
// column l % 16.
__device__ __forceinline__ floatx4 mfma16_bf16(const ushortx8 &a, const ushortx8 &b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// 32x32x16 bf16 -> fp32. Lane l supplies row l % 32, contraction slots
// 8*(l/32) .. +7; result register r holds row 8*(r/4) + 4*(l/32) + r%4 of
// column l % 32.
__device__ __forceinline__ floatx16 mfma32_bf16(const ushortx8 &a, const ushortx8 &b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// ------------------------------------------------------------------ misc
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Max over a wavefront (64 lanes) with cross-lane shuffles.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}


// ------------------------------------------------------------ fp64 lanes
// A DPP move of an fp64 value (both halves with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __double2loint(v), hi = __double2hiint(v);
  return __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false),
                          __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of 8 lanes; every lane gets the bitwise same sum.
__device__ __forceinline__ double group8_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);  // row_half_mirror: lane i with lane 7 - i
  return v;
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}

// Sum over the whole wave (every lane active), the same bits in every lane:
// DPP within rows of 16 lanes, then the four row sums read as scalars.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = group8_sum(v);
  v += dpp_f64<0x140>(v);  // row_mirror: lane i with lane 15 - i
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

}  // namespace metis

// ------------------------------------------------------------------ host
namespace metis_host {

// Bump allocator over a caller workspace; every carve is 256-byte aligned.
struct Carver {
  char *base;
  size_t off;
  explicit Carver(void *b) : base((char *)b), off(0) {}
  template <typename T> T *take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T *p = base ? (T *)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return (off + 255) & ~(size_t)255; }
};

}  // namespace metis_host

// Copy `count` elements src[si(i)] -> dst[di(i)] (dst usually LDS) with the
// whole block: each thread issues PER loads before the first of them is
// used, so a small matrix arrives in count / (PER * blockDim.x) memory round
// trips instead of one round trip per element a thread handles.
template <int PER, typename T, typename SrcIdx, typename DstIdx>
__device__ __forceinline__ void stage_batched(T *dst, const T *__restrict__ src, int count, SrcIdx si, DstIdx di) {
  const int t = threadIdx.x, nt = blockDim.x;
  for (int base = 0; base < count; base += PER * nt) {
    T v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + t + u * nt;
      v[u] = i < count ? src[si(i)] : T(0);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = base + t + u * nt;
      if (i < count) dst[di(i)] = v[u];
    }
  }
}

#define METIS_LAUNCH_CHECK()                                \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return METIS_ERR_HIP; \
  } while (0)
