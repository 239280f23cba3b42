// Standalone block FP4 codec: fp4_block_quant / fp4_block_dequant.
//
// Pure streaming passes (HBM bound): each thread owns whole blocks, so no
// cross-lane reduction is needed for the block max. The transposed variant
// reads a column strip with lanes spread over consecutive columns (coalesced
// reads) and writes four consecutive blocks of one output row per thread.
#include "common.hpp"

using namespace metis;

namespace {

constexpr int kThreads = 256;
constexpr int kTransBytes = 128;  // code bytes of an output row per thread in the transposed kernel

// Quantize one block held in registers. Returns the scale byte; codes are
// packed into `packed` (B/2 bytes, element 2j in the low nibble of byte j).
template <int B, bool NV>
__device__ __forceinline__ uint32_t quant_block(const float (&v)[B], float s_t, uint32_t (&packed)[B / 8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < B; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t scale_byte;
  if (!NV) {
    const int se = mx_shared_exponent(amax);
    scale_byte = (uint32_t)(se + 127);
    e2m1_pack_scaled<B>(v, pow2_f32(se), packed);
  } else {
    const float d = 6.0f * s_t;
    scale_byte = e4m3_rne_sat(__fdiv_rn(amax, d));
    const float den = e4m3_value(scale_byte) * s_t;
    // a zero scale leaves only the signs (v * 0 keeps the sign of v)
    float q[B];
#pragma unroll
    for (int i = 0; i < B; ++i) q[i] = scale_byte ? __fdiv_rn(v[i], den) : v[i] * 0.0f;
    e2m1_pack<B>(q, packed);
  }
  return scale_byte;
}

template <typename T>
__global__ void fill_u32_kernel(uint32_t *p, uint32_t v, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Max |x| over a rows x cols matrix into *out (as fp32 bits; non-negative
// floats order like their bit patterns, so an integer max is exact and
// independent of the order of arrival).
template <typename T>
__global__ void amax_kernel(const T *__restrict__ x, int64_t rows, int64_t cols, int64_t ldx, uint32_t *out) {
  // workgroup b takes rows b, b + gridDim.x, ...; its threads stride along
  // the row (coalesced loads, no index division)
  float m = 0.0f;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T *row = x + r * ldx;
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) m = fmaxf(m, fabsf(load_f32(row + c)));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(m));
}

template <typename T, bool NV>
__global__ void __launch_bounds__(kThreads) quant_rows_kernel(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                              int64_t ldx, uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales, const uint32_t *amax_bits,
                                                              float *tensor_scale) {
  constexpr int B = NV ? 16 : 32;
  const int64_t per_row = cols / B;
  const int64_t b = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  float s_t = 1.0f;
  if (NV) {
    s_t = nv_tensor_scale(__uint_as_float(*amax_bits));
    if (b == 0) *tensor_scale = s_t;
  }
  if (b >= rows * per_row) return;
  const int64_t r = b / per_row, cb = b - r * per_row;
  const T *src = x + r * ldx + cb * B;
  float v[B];
#pragma unroll
  for (int i = 0; i < B; ++i) v[i] = load_f32(src + i);
  uint32_t packed[B / 8];
  const uint32_t sb = quant_block<B, NV>(v, s_t, packed);
  uint32_t *dst = (uint32_t *)(codes + r * (cols / 2) + cb * (B / 2));
#pragma unroll
  for (int w = 0; w < B / 8; ++w) dst[w] = packed[w];
  scales[b] = (uint8_t)sb;
}

// out = x^T (cols x rows), blocks along rows. Thread (c, g) quantizes the
// 256 / B consecutive row blocks g (256 / B).. of column c: 128 bytes of codes
// of output row c, a whole cache line. They are staged in the thread's own
// row of LDS and written together at the end, so the line's pieces reach the
// L2 back to back (stored as each block was done, the L2 wrote many lines
// back in pieces).
template <typename T, bool NV>
__global__ void __launch_bounds__(kThreads) quant_cols_kernel(const T *__restrict__ x, int64_t rows, int64_t cols,
                                                              int64_t ldx, uint8_t *__restrict__ codes,
                                                              uint8_t *__restrict__ scales, const uint32_t *amax_bits,
                                                              float *tensor_scale) {
  constexpr int B = NV ? 16 : 32;
  constexpr int TB = kTransBytes * 2 / B;  // row blocks per thread
  constexpr int W = B / 8;                  // code words per block
  __shared__ uint32_t cst[kThreads][TB * W + 1];  // odd row stride: no bank conflicts
  __shared__ uint8_t sst[kThreads][TB];
  const int t = threadIdx.x;
  const int64_t c = blockIdx.x * (int64_t)kThreads + t;
  const int64_t g = blockIdx.y;
  float s_t = 1.0f;
  if (NV) {
    s_t = nv_tensor_scale(__uint_as_float(*amax_bits));
    if (c == 0 && g == 0) *tensor_scale = s_t;
  }
  if (c >= cols) return;  // each thread touches only its own LDS rows: no barrier follows
  const int64_t nblk = rows / B, blk0 = g * TB;
  const int nb = (int)min<int64_t>(TB, nblk - blk0);
#pragma unroll 1
  for (int j = 0; j < nb; ++j) {
    const int64_t blk = blk0 + j;
    float v[B];
#pragma unroll
    for (int i = 0; i < B; ++i) v[i] = load_f32(x + (blk * B + i) * ldx + c);
    uint32_t packed[W];
    const uint32_t sb = quant_block<B, NV>(v, s_t, packed);
#pragma unroll
    for (int w = 0; w < W; ++w) cst[t][j * W + w] = packed[w];
    sst[t][j] = (uint8_t)sb;
  }
  uint32_t *dst = (uint32_t *)(codes + c * (rows / 2) + blk0 * (B / 2));  // 16-byte aligned (rows % 32 == 0)
  if (nb == TB) {
#pragma unroll
    for (int q = 0; q < TB * W / 4; ++q)
      ((uint4 *)dst)[q] = uint4{cst[t][4 * q], cst[t][4 * q + 1], cst[t][4 * q + 2], cst[t][4 * q + 3]};
  } else {
    for (int w = 0; w < nb * W; ++w) dst[w] = cst[t][w];
  }
  for (int j = 0; j < nb; ++j) scales[c * nblk + blk0 + j] = sst[t][j];
}

template <bool NV>
__global__ void __launch_bounds__(kThreads) dequant_kernel(const uint8_t *__restrict__ codes,
                                                           const uint8_t *__restrict__ scales, const float *tensor_scale,
                                                           int64_t rows, int64_t cols, float *__restrict__ y,
                                                           int64_t ldy) {
  constexpr int B = NV ? 16 : 32;
  const int64_t per_row = cols / B;
  const int64_t b = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (b >= rows * per_row) return;
  const int64_t r = b / per_row, cb = b - r * per_row;
  const uint32_t sb = scales[b];
  const uint32_t *src = (const uint32_t *)(codes + r * (cols / 2) + cb * (B / 2));
  float *dst = y + r * ldy + cb * B;
  if (!NV) {
    const int se = (int)sb - 127;
#pragma unroll
    for (int w = 0; w < B / 8; ++w) {
      const uint32_t p = src[w];
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[w * 8 + j] = ldexpf(e2m1_value((p >> (4 * j)) & 15u), se);
    }
  } else {
    const float sv = e4m3_value(sb);
    const float st = *tensor_scale;
#pragma unroll
    for (int w = 0; w < B / 8; ++w) {
      const uint32_t p = src[w];
      // value(code) * value(scale) is exact in fp32; one rounding by s_t
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[w * 8 + j] = (e2m1_value((p >> (4 * j)) & 15u) * sv) * st;
    }
  }
}

template <typename T, bool NV>
metis_status_t launch_quant(const T *x, int64_t rows, int64_t cols, int64_t ldx, int transpose, metis_fp4_t *out,
                            uint32_t *amax_ws, hipStream_t stream) {
  if (NV) {
    fill_u32_kernel<int><<<1, 64, 0, stream>>>(amax_ws, 0u, 1);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(2048, rows));
    amax_kernel<T><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, amax_ws);
  }
  constexpr int B = NV ? 16 : 32;
  if (!transpose) {
    const int64_t nblocks = rows * (cols / B);
    quant_rows_kernel<T, NV><<<(unsigned)cdiv(nblocks, kThreads), kThreads, 0, stream>>>(
        x, rows, cols, ldx, out->codes, out->scales, amax_ws, out->tensor_scale);
  } else {
    dim3 grid((unsigned)cdiv(cols, kThreads), (unsigned)cdiv(rows / B, kTransBytes * 2 / B));
    quant_cols_kernel<T, NV><<<grid, kThreads, 0, stream>>>(x, rows, cols, ldx, out->codes, out->scales, amax_ws,
                                                            out->tensor_scale);
  }
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

}  // namespace

extern "C" size_t fp4_block_quant_workspace_bytes(int64_t rows, int64_t cols, metis_fmt_t fmt) {
  (void)rows;
  (void)cols;
  return fmt == METIS_NVFP4 ? 256 : 0;
}

extern "C" metis_status_t fp4_block_quant(const void *x, metis_dtype_t dt, int64_t rows, int64_t cols, int64_t ldx,
                                          int32_t transpose, metis_fp4_t *out, void *ws, size_t ws_bytes,
                                          hipStream_t stream) {
  if (!out || rows < 0 || cols < 0 || ldx < cols || (transpose != 0 && transpose != 1)) return METIS_ERR_INVALID;
  if (dt != METIS_F32 && dt != METIS_BF16) return METIS_ERR_INVALID;
  if (out->fmt != METIS_MXFP4 && out->fmt != METIS_NVFP4) return METIS_ERR_INVALID;
  const bool nv = out->fmt == METIS_NVFP4;
  const int64_t B = nv ? 16 : 32;
  const int64_t blocked = transpose ? rows : cols;
  if (blocked % B) return METIS_ERR_INVALID;
  out->rows = transpose ? cols : rows;
  out->cols = transpose ? rows : cols;
  if (rows == 0 || cols == 0) return METIS_OK;
  if (!x || !out->codes || !out->scales) return METIS_ERR_INVALID;
  if (((uintptr_t)out->codes) & 3) return METIS_ERR_INVALID;  // codes are written as 32-bit words
  if (nv && !out->tensor_scale) return METIS_ERR_INVALID;
  if (nv && (!ws || ws_bytes < fp4_block_quant_workspace_bytes(rows, cols, (metis_fmt_t)out->fmt))) return METIS_ERR_WORKSPACE;
  uint32_t *amax_ws = (uint32_t *)ws;
  if (dt == METIS_F32) {
    return nv ? launch_quant<float, true>((const float *)x, rows, cols, ldx, transpose, out, amax_ws, stream)
              : launch_quant<float, false>((const float *)x, rows, cols, ldx, transpose, out, amax_ws, stream);
  }
  return nv ? launch_quant<unsigned short, true>((const unsigned short *)x, rows, cols, ldx, transpose, out, amax_ws,
                                                 stream)
            : launch_quant<unsigned short, false>((const unsigned short *)x, rows, cols, ldx, transpose, out, amax_ws,
                                                  stream);
}

extern "C" metis_status_t fp4_block_dequant(const metis_fp4_t *in, float *y, int64_t ldy, hipStream_t stream) {
  if (!in || in->rows < 0 || in->cols < 0 || ldy < in->cols) return METIS_ERR_INVALID;
  if (in->fmt != METIS_MXFP4 && in->fmt != METIS_NVFP4) return METIS_ERR_INVALID;
  const bool nv = in->fmt == METIS_NVFP4;
  const int64_t B = nv ? 16 : 32;
  if (in->cols % B) return METIS_ERR_INVALID;
  if (in->rows == 0 || in->cols == 0) return METIS_OK;
  if (!y || !in->codes || !in->scales || (nv && !in->tensor_scale)) return METIS_ERR_INVALID;
  if (((uintptr_t)in->codes) & 3) return METIS_ERR_INVALID;
  const int64_t nblocks = in->rows * (in->cols / B);
  const unsigned grid = (unsigned)cdiv(nblocks, kThreads);
  if (nv)
    dequant_kernel<true><<<grid, kThreads, 0, stream>>>(in->codes, in->scales, in->tensor_scale, in->rows, in->cols, y,
                                                        ldy);
  else
    dequant_kernel<false><<<grid, kThreads, 0, stream>>>(in->codes, in->scales, nullptr, in->rows, in->cols, y, ldy);
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

extern "C" const char *metis_status_str(metis_status_t s) {
  switch (s) {
    case METIS_OK: return "METIS_OK";
    case METIS_ERR_INVALID: return "METIS_ERR_INVALID";
    case METIS_ERR_UNSUPPORTED: return "METIS_ERR_UNSUPPORTED";
    case METIS_ERR_WORKSPACE: return "METIS_ERR_WORKSPACE";
    case METIS_ERR_HIP: return "METIS_ERR_HIP";
    case METIS_ERR_TOO_LARGE: return "METIS_ERR_TOO_LARGE";
  }
  return "METIS_ERR_UNKNOWN";
}

extern "C" int32_t metis_abi_version(void) { return 2; }
