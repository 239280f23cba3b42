// W4A4G4 linear layer on quantized split operands ("Metis: Training LLMs with
// FP4 Quantization", abstract: FP4 weights, activations and gradients).
//
// Each GEMM is C = A_hat B_hat^T with, for a split operand in the orientation
// it is used in, A_hat = R + G diag(S) F^T (R: residual blocked along the
// contraction axis T; F: the factor along T, quantized along T; G: the factor
// along the output axis). Expanding both operands:
//   C = Ra Rb^T + (Ra Fb Sb) Gb^T + Ga [Sa (Fa^T Rb^T + (Fa^T Fb) Sb Gb^T)]
//     = Ra Rb^T + L1 L2^T,
//   L1 = [P_hi  P_lo  Ga  Ga],  L2 = [Gb  Gb  Q_hi  Q_lo],
//   P  = Ra Fb diag(Sb),        Q  = (Rb Fa + Gb diag(Sb) (Fa^T Fb)^T) diag(Sa).
// G values are FP4 codes times power-of-two scales, exact in bf16; P and Q are
// carried as bf16 hi + lo (16 significant bits), so the bf16 MFMA correction
// is fp32-accurate. Kernels:
//   skinny_kernel  P, Q and Fa^T Fb on the scaled FP4 MFMA (split-K partials)
//   panel_kernel   sums the partials and writes the bf16 panels L1, L2
//   gemm_mx_kernel Ra Rb^T on v_mfma_scale_f32_32x32x64_f8f6f4 (256 x 256
//                  tiles, a four-stage LDS ring filled by asynchronous
//                  global-to-LDS loads), then + L1 L2^T on bf16 MFMA into the
//                  same accumulators, its panels streamed through the same
//                  ring, then one fp32 store (K a multiple of 512).
//   gemm_mx8_kernel the same product for any K (register-staged loads,
//                  correction panels staged in the epilogue).
//   gemm_nv_kernel the NVFP4 form: E2M1 x E4M3 decoded exactly to fp16 in the
//                  LDS staging (hardware FP4 conversion, one packed fp16
//                  multiply by the block scale), fp16 MFMA (gfx950's scaled
//                  MFMA takes only E8M0 scales per 32 elements), tensor
//                  scales in the epilogue.
//   skinny_nv_kernel, panel_kernel<true>: the NVFP4 forms of the first two.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.hpp"

using namespace metis;

namespace {

// ---------------------------------------------------------------- operands
// One side of an NT GEMM: residual R (rows x T) blocked along T, factors.
struct Side {
  const metis_fp4_t *R;
  const metis_fp4_t *F;  // contracted factor, k x T (blocked along T)
  const metis_fp4_t *G;  // outer factor, k x rows (blocked along rows)
  const float *S;
  int64_t rows, T;
  int k;
};

bool make_side(const metis_split_t *s, bool transposed, Side &out) {
  out.R = transposed ? &s->Rt_q : &s->R_q;
  out.rows = transposed ? s->n : s->m;
  out.T = transposed ? s->m : s->n;
  if (out.rows < 0 || out.T < 0) return false;
  if (out.rows > 0 && out.T > 0 && (!out.R->codes || !out.R->scales)) return false;
  out.k = s->k;
  out.S = s->S;
  out.F = transposed ? &s->Ut_q : &s->Vt_q;
  out.G = transposed ? &s->Vt_q : &s->Ut_q;
  if (s->k > 0 && (!s->S || !out.F->codes || !out.F->scales || !out.G->codes || !out.G->scales)) return false;
  if (s->k > 0 && (out.F->rows != s->k || out.F->cols != out.T || out.G->rows != s->k || out.G->cols != out.rows ||
                   out.rows % 32 || (((uintptr_t)out.F->codes) & 15)))
    return false;
  return true;
}

struct GemmPlan {
  int64_t ra, rb, T;
  int ka, kb, rp;
  int ks_p, ks_q, ks_c;          // split-K counts of the skinny products
  int64_t tc_p, tc_q, tc_c;      // T per split (multiple of 128)
  float *ppart, *qpart, *cpart;  // partials
  float *cross;                  // ka x kb, the summed cpart
  unsigned short *l1, *l2;       // panels
  size_t bytes;
};

// Split-K of a skinny product over row blocks of 128: at least 256
// workgroups when the contraction allows, each split at least four stages of
// 256 elements (chunk a multiple of 256).
int64_t pick_split(int64_t rows, int64_t T, int64_t &chunk) {
  const int64_t row_blocks = std::max<int64_t>(1, cdiv(rows, 128));
  int64_t want = std::max<int64_t>(1, cdiv(256, row_blocks));
  want = std::min<int64_t>(want, std::max<int64_t>(1, T / 1024));
  chunk = round_up(cdiv(T, want), 256);
  return cdiv(T, chunk);
}

GemmPlan make_gemm_plan(int64_t ra, int64_t rb, int64_t T, int ka, int kb, void *ws) {
  GemmPlan p;
  p.ra = ra; p.rb = rb; p.T = T; p.ka = ka; p.kb = kb;
  p.rp = (int)round_up(2 * ka + 2 * kb, 64);
  p.ks_p = kb ? (int)pick_split(ra, T, p.tc_p) : 0;
  p.ks_q = ka ? (int)pick_split(rb, T, p.tc_q) : 0;
  p.ks_c = (ka && kb) ? (int)pick_split(ka, T, p.tc_c) : 0;
  metis_host::Carver c(ws);
  p.ppart = c.take<float>((size_t)p.ks_p * ra * kb);
  p.qpart = c.take<float>((size_t)p.ks_q * rb * ka);
  p.cpart = c.take<float>((size_t)p.ks_c * ka * kb);
  p.cross = c.take<float>((size_t)ka * kb);
  p.l1 = c.take<unsigned short>((size_t)ra * p.rp);
  p.l2 = c.take<unsigned short>((size_t)rb * p.rp);
  p.bytes = c.bytes();
  return p;
}

// Packed FP4 view of an MFMA operand: 32 codes (16 bytes) in 4 dwords.
__device__ __forceinline__ intx8 fp4x32(const uint4 v) { return intx8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

__device__ __forceinline__ floatx16 mfma_fp4(const uint4 a, const uint4 b, int sa, int sb, floatx16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4x32(a), fp4x32(b), c, 4, 4, 0, sa, 0, sb);
}

// ================================================================== skinny
// out[s] (rows x cols) = NT(A (rows x T), B (cols x T)) over T-chunk s, both
// MXFP4. One wave: 32 rows x (32 * NCT) columns, 512 contraction elements
// per step: lane (r, h) owns elements [t0 + 256 h, t0 + 256 h + 256) of its
// row, eight scale blocks, read as eight 16-byte code pieces and (when a row's
// scale count is a multiple of four) two 32-bit scale words. MFMA c of a step
// takes block c of every lane's span from A and from B alike, so the K slots
// of the two operands line up; its scale byte is picked from the word by
// opsel. Blocks past the chunk read zero codes (any scale).
__device__ __forceinline__ void skinny_load_span(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                                 int64_t row, bool rok, int64_t e0, int64_t t_end, int64_t T,
                                                 bool word_scales, uint4 (&c)[8], uint32_t (&w)[2]) {
  const int64_t nb = T / 32;
  const uint4 *p = (const uint4 *)(codes + row * (T / 2) + e0 / 2);
#pragma unroll
  for (int q = 0; q < 8; ++q) c[q] = (rok && e0 + 32 * q < t_end) ? p[q] : uint4{0u, 0u, 0u, 0u};
  const uint8_t *ps = scales + row * nb + e0 / 32;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (word_scales) {
      w[q] = (rok && e0 + 128 * q < t_end) ? *(const uint32_t *)(ps + 4 * q) : 0x7F7F7F7Fu;
    } else {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = rok && e0 + 32 * (4 * q + i) < t_end;
        v |= (ok ? (uint32_t)ps[4 * q + i] : 127u) << (8 * i);
      }
      w[q] = v;
    }
  }
}

template <int C>
__device__ __forceinline__ floatx16 skinny_mfma(const uint4 &a, const uint4 &b, uint32_t sa, uint32_t sb, floatx16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4x32(a), fp4x32(b), acc, 4, 4, C % 4, (int)sa, C % 4,
                                                          (int)sb);
}

template <int NCT>
__global__ void __launch_bounds__(64)
    skinny_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t rows,
                  const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs, int cols, int64_t T, int64_t chunk,
                  float *__restrict__ out) {
  const int lane = threadIdx.x;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + r;
  const int s = blockIdx.y;
  const int64_t t_beg = (int64_t)s * chunk, t_end = std::min<int64_t>(T, t_beg + chunk);
  const bool word_scales = ((T / 32) & 3) == 0;
  floatx16 acc[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  const bool rok = row < rows;
  for (int64_t t0 = t_beg; t0 < t_end; t0 += 512) {
    const int64_t e0 = t0 + 256 * h;
    uint4 a[8], b[NCT][8];
    uint32_t sa[2], sb[NCT][2];
    skinny_load_span(ac, as, row, rok, e0, t_end, T, word_scales, a, sa);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int col = j * 32 + r;
      skinny_load_span(bc, bs, col, col < cols, e0, t_end, T, word_scales, b[j], sb[j]);
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      acc[j] = skinny_mfma<0>(a[0], b[j][0], sa[0], sb[j][0], acc[j]);
      acc[j] = skinny_mfma<1>(a[1], b[j][1], sa[0], sb[j][0], acc[j]);
      acc[j] = skinny_mfma<2>(a[2], b[j][2], sa[0], sb[j][0], acc[j]);
      acc[j] = skinny_mfma<3>(a[3], b[j][3], sa[0], sb[j][0], acc[j]);
      acc[j] = skinny_mfma<0>(a[4], b[j][4], sa[1], sb[j][1], acc[j]);
      acc[j] = skinny_mfma<1>(a[5], b[j][5], sa[1], sb[j][1], acc[j]);
      acc[j] = skinny_mfma<2>(a[6], b[j][6], sa[1], sb[j][1], acc[j]);
      acc[j] = skinny_mfma<3>(a[7], b[j][7], sa[1], sb[j][1], acc[j]);
    }
  }
  float *o = out + (int64_t)s * rows * cols;
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int col = j * 32 + r;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t orow = (int64_t)blockIdx.x * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
      if (orow < rows && col < cols) o[orow * cols + col] = acc[j][q];
    }
  }
}

// Eight E2M1 codes (element 2p in the low nibble of byte p, 2p + 1 in the
// high one) times one block scale, as fp16. The byte selector of the FP4
// conversion is an immediate, hence the four spelled-out calls.
__device__ __forceinline__ halfx8 fp4x8_to_f16(uint32_t word, halfx2 scale) {
  const halfx2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * scale;
  const halfx2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * scale;
  const halfx2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * scale;
  const halfx2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * scale;
  return halfx8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// NVFP4 variant: both operands decoded exactly to fp16 by the hardware FP4
// conversion and one packed multiply by the E4M3 block scale (each product
// has at most five significant bits and lies in [2^-10, 2688]) and multiplied
// on the fp16 MFMA; the two tensor scales multiply the fp32 result once. One
// wave: 32 rows x 32*NCT columns; per 32-element step lane (r, h) decodes
// block h (16 elements) of its row and feeds its first and second 8 values to
// two 32x32x16 MFMAs.
__device__ __forceinline__ void nv_decode16(const uint2 codes, uint32_t sbyte, halfx8 &lo8, halfx8 &hi8) {
  const _Float16 sv = (_Float16)e4m3_value(sbyte);  // exact: every E4M3 value is an fp16 value
  const halfx2 s2 = {sv, sv};
  lo8 = fp4x8_to_f16(codes.x, s2);
  hi8 = fp4x8_to_f16(codes.y, s2);
}

template <int NCT>
__global__ void __launch_bounds__(64)
    skinny_nv_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, const float *__restrict__ ats,
                     int64_t rows, const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs,
                     const float *__restrict__ bts, int cols, int64_t T, int64_t chunk, float *__restrict__ out) {
  const int lane = threadIdx.x;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + r;
  const int s = blockIdx.y;
  const int64_t t_beg = (int64_t)s * chunk, t_end = std::min<int64_t>(T, t_beg + chunk);
  const int64_t nb = T / 16;
  floatx16 acc[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  const bool rok = row < rows;
  const halfx8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t t0 = t_beg; t0 < t_end; t0 += 32) {
    const int64_t e0 = t0 + h * 16;
    halfx8 a0 = z8, a1 = z8;
    if (rok && e0 < t_end) nv_decode16(*(const uint2 *)(ac + row * (T / 2) + e0 / 2), as[row * nb + e0 / 16], a0, a1);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int col = j * 32 + r;
      halfx8 b0 = z8, b1 = z8;
      if (col < cols && e0 < t_end)
        nv_decode16(*(const uint2 *)(bc + (int64_t)col * (T / 2) + e0 / 2), bs[(int64_t)col * nb + e0 / 16], b0, b1);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc[j], 0, 0, 0);
    }
  }
  const float sc = ats[0] * bts[0];
  float *o = out + (int64_t)s * rows * cols;
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int col = j * 32 + r;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t orow = (int64_t)blockIdx.x * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
      if (orow < rows && col < cols) o[orow * cols + col] = acc[j][q] * sc;
    }
  }
}

// =================================================================== panels
// cross = sum of the ks split-K slabs of Fa^T Fb (fixed order).
__global__ void cross_reduce_kernel(const float *__restrict__ cpart, int ks, int count, float *__restrict__ cross) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= count) return;
  float v = 0.0f;
  for (int s = 0; s < ks; ++s) v += cpart[(int64_t)s * count + e];
  cross[e] = v;
}

// Blocks [0, ceil(ra / 32)) build 32 rows of L1 each, the following blocks 32
// rows of L2. The factor values, P and Q of the block's rows are formed in LDS
// first (factor codes read along the rows, partial sums along the columns),
// then each panel row is written contiguously. The G columns of the panels
// hold e2m1 * block scale, which bf16 represents exactly; for NVFP4 the G
// tensor scale is folded into the partner column (P for Gb, Q for Ga) before
// its hi/lo split. Every global read is batched (a thread's loads of one
// phase are in flight together), since the block is bound by load latency.
constexpr int kPanelRows = 32;
constexpr int kPanelThreads = 256;
// elements per thread of a kPanelRows x k block, k <= KM (64 or 96)
template <int KM>
constexpr int panel_per() { return (kPanelRows * KM + kPanelThreads - 1) / kPanelThreads; }

// dst(i, sum) for i < count, sum = src[i] + src[stride + i] + ... over
// nslabs slabs in slab order; four slabs' loads in flight at a time.
template <int kPanelPer, typename Store>
__device__ __forceinline__ void panel_sum_slabs(const float *__restrict__ src, int64_t stride, int nslabs, int count,
                                                Store store) {
  const int t = threadIdx.x;
  float acc[kPanelPer];
#pragma unroll
  for (int v = 0; v < kPanelPer; ++v) acc[v] = 0.0f;
  int s = 0;
  for (; s + 4 <= nslabs; s += 4) {
    float x[4][kPanelPer];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < kPanelPer; ++v) {
        const int i = t + v * kPanelThreads;
        x[u][v] = i < count ? src[(int64_t)(s + u) * stride + i] : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < kPanelPer; ++v) acc[v] += x[u][v];
  }
  for (; s < nslabs; ++s) {
    float x[kPanelPer];
#pragma unroll
    for (int v = 0; v < kPanelPer; ++v) {
      const int i = t + v * kPanelThreads;
      x[v] = i < count ? src[(int64_t)s * stride + i] : 0.0f;
    }
#pragma unroll
    for (int v = 0; v < kPanelPer; ++v) acc[v] += x[v];
  }
#pragma unroll
  for (int v = 0; v < kPanelPer; ++v) {
    const int i = t + v * kPanelThreads;
    if (i < count) store(i, acc[v]);
  }
}

// Decoded values of a k x rows factor matrix at rows [r0, r0 + nr), columns
// c < k, in two parts so other loads can be in flight between them:
// load() issues every code and scale load of the thread at once (from a
// valid index, element (0, r0) when out of range, none behind a branch);
// decode() then calls store(c, r, e2m1 * block scale). k = 0 (an unsplit
// side, possibly without buffers) loads and stores nothing.
template <bool NV, int KM>
struct PanelFactor {
  static constexpr int kPanelPer = panel_per<KM>();
  uint32_t cb[kPanelPer], sb[kPanelPer];
  __device__ __forceinline__ void load(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                                       int64_t rows, int k, int64_t r0, int nr) {
    constexpr int B = NV ? 16 : 32;
    if (k <= 0) return;
#pragma unroll
    for (int v = 0; v < kPanelPer; ++v) {
      const int e = threadIdx.x + v * kPanelThreads, c = e / kPanelRows, r = e - c * kPanelRows;
      const bool ok = c < k && r < nr;
      const int64_t cc = ok ? c : 0, i = r0 + (ok ? r : 0);
      cb[v] = codes[cc * (rows / 2) + i / 2];
      sb[v] = scales[cc * (rows / B) + i / B];
    }
  }
  template <typename Store>
  __device__ __forceinline__ void decode(int k, int64_t r0, int nr, Store store) {
    if (k <= 0) return;
    // the decode stays here (the compiler would otherwise hoist it, and the
    // wait for these loads, above the loads issued in between)
#pragma unroll
    for (int v = 0; v < kPanelPer; ++v) __asm__ volatile("" : "+v"(cb[v]), "+v"(sb[v]));
#pragma unroll
    for (int v = 0; v < kPanelPer; ++v) {
      const int e = threadIdx.x + v * kPanelThreads, c = e / kPanelRows, r = e - c * kPanelRows;
      if (c < k && r < nr) {
        const uint32_t code = ((r0 + r) & 1) ? (cb[v] >> 4) : (cb[v] & 15u);
        const float val = NV ? e2m1_value(code) * e4m3_value(sb[v]) : ldexpf(e2m1_value(code), (int)sb[v] - 127);
        store(c, r, val);
      }
    }
  }
};

// n / d for 0 <= n, n * d < 2^32 and d > 0: the high half of n * m with
// m = floor((2^32 - 1) / d) + 1 (then m d - 2^32 < d, which keeps the
// quotient exact in that range). d = 1 (m = 2^32 does not fit) returns n;
// d = 0 is never divided by.
struct FastDiv {
  uint32_t d, m;
  __device__ explicit FastDiv(int dd) : d((uint32_t)dd), m(dd > 1 ? 0xFFFFFFFFu / (uint32_t)dd + 1u : 0u) {}
  __device__ __forceinline__ int div(int n) const { return d == 1u ? n : (int)__umulhi((uint32_t)n, m); }
  __device__ __forceinline__ int mod(int n) const { return n - div(n) * (int)d; }
};

// Rows [0, nr) of a panel (row stride rp, a multiple of 64) from value(r, c),
// eight columns per 16-byte store. Wave w takes the 64-column groups w,
// w + 4, ...; its lane (p, rr) writes piece p of the group on rows rr,
// rr + 8, ... (eight whole 128-byte row pieces per store instruction). A
// panel's column sections are 64 wide when k = 64, so value() takes one
// path per wave.
template <typename Value>
__device__ __forceinline__ void panel_write_rows(unsigned short *__restrict__ dst, int nr, int rp, Value value) {
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int g = w; g * 64 < rp; g += kPanelThreads / 64) {
    const int c0 = 64 * g + 8 * (lane & 7);
    for (int r = lane >> 3; r < nr; r += 8) {
      ushortx8 v;
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = value(r, c0 + u);
      *(ushortx8 *)(dst + (int64_t)r * rp + c0) = v;
    }
  }
}

template <bool NV, int KM>
__global__ void __launch_bounds__(kPanelThreads)
    panel_kernel(int64_t ra, int64_t rb, int ka, int kb, int rp, const float *__restrict__ ppart, int ks_p,
                 const float *__restrict__ qpart, int ks_q, const float *__restrict__ cross_g,
                 const float *__restrict__ Sa, const float *__restrict__ Sb, const uint8_t *__restrict__ ga_c,
                 const uint8_t *__restrict__ ga_s, const float *__restrict__ ga_t, const uint8_t *__restrict__ gb_c,
                 const uint8_t *__restrict__ gb_s, const float *__restrict__ gb_t, unsigned short *__restrict__ l1,
                 unsigned short *__restrict__ l2) {
  constexpr int R = kPanelRows, KP = KM + 1, PER = panel_per<KM>();
  constexpr int CPER = (KM * KM + kPanelThreads - 1) / kPanelThreads;  // cross elements per thread
  __shared__ float cross[KM][KP];
  __shared__ float fv[R][KP];  // L1: P (summed partials); L2: Gb values
  __shared__ float gv[R][KP];  // L1: Ga values; L2: Gb values * tensor scale * Sb
  __shared__ float qv[R][KP];  // L2: Q
  __shared__ float sa_s[KM], sb_s[KM], ts_s[2];
  const int t = threadIdx.x;
  const int64_t l1_blocks = (ra + R - 1) / R;
  if (t < ka) sa_s[t] = Sa[t];
  if (t < kb) sb_s[t] = Sb[t];
  if (t == 0) {
    ts_s[0] = (NV && ka) ? ga_t[0] : 1.0f;  // Ga tensor scale, carried by Q
    ts_s[1] = (NV && kb) ? gb_t[0] : 1.0f;  // Gb tensor scale, carried by P
  }
  if ((int64_t)blockIdx.x < l1_blocks) {
    const int64_t i0 = (int64_t)blockIdx.x * R;
    const int nr = (int)min<int64_t>(R, ra - i0);
    PanelFactor<NV, KM> fa;
    fa.load(ga_c, ga_s, ra, ka, i0, nr);  // in flight during the slab sums
    const FastDiv dkb(kb);
    panel_sum_slabs<PER>(ppart + i0 * kb, ra * kb, ks_p, nr * kb, [&](int i, float v) {
      const int r = dkb.div(i);
      fv[r][i - r * kb] = v;
    });
    fa.decode(ka, i0, nr, [&](int c, int r, float v) { gv[r][c] = v; });
    __syncthreads();
    const float fold_b = ts_s[1];
    panel_write_rows(l1 + i0 * rp, nr, rp, [&](int r, int c) -> unsigned short {
      if (c < 2 * kb) {
        unsigned short hi, lo;
        const int d = c < kb ? c : c - kb;
        split_bf16(fv[r][d] * sb_s[d] * fold_b, hi, lo);
        return c < kb ? hi : lo;
      }
      c -= 2 * kb;
      return c < 2 * ka ? f32_to_bf16(gv[r][c < ka ? c : c - ka]) : (unsigned short)0;
    });
  } else {
    const int64_t j0 = ((int64_t)blockIdx.x - l1_blocks) * R;
    const int nr = (int)min<int64_t>(R, rb - j0);
    // the factor codes, the summed Fa^T Fb and the Q partials of the block's
    // rows are all requested before the first of them is used
    PanelFactor<NV, KM> fb;
    fb.load(gb_c, gb_s, rb, kb, j0, nr);
    const int ncross = (ka && kb) ? ka * kb : 0;
    float xc[CPER];
#pragma unroll
    for (int u = 0; u < CPER; ++u) {
      const int i = t + u * kPanelThreads;
      xc[u] = ncross ? cross_g[i < ncross ? i : 0] : 0.0f;  // (a uniform test: no cross for an unsplit side)
    }
    const FastDiv dka(ka), dkb(kb);
    panel_sum_slabs<PER>(qpart + j0 * ka, rb * ka, ks_q, nr * ka, [&](int i, float v) {
      const int r = dka.div(i);
      qv[r][i - r * ka] = v;
    });
    // the stores stay here (the compiler would otherwise hoist them, and the
    // wait for these loads, above the slab loads)
#pragma unroll
    for (int u = 0; u < CPER; ++u) __asm__ volatile("" : "+v"(xc[u]));
#pragma unroll
    for (int u = 0; u < CPER; ++u) {
      const int i = t + u * kPanelThreads;
      if (i < ncross) {
        const int c = dkb.div(i);
        cross[c][i - c * kb] = xc[u];
      }
    }
    fb.decode(kb, j0, nr, [&](int d, int r, float v) { fv[r][d] = v; });
    __syncthreads();
    const float fold_a = ts_s[0], tsb = NV ? ts_s[1] : 1.0f;
    for (int e = t; e < nr * kb; e += kPanelThreads) {
      const int r = dkb.div(e), d = e - r * kb;
      gv[r][d] = fv[r][d] * tsb * sb_s[d];
    }
    __syncthreads();
    // Q[r][cc] += sum_d gv[r][d] cross[cc][d]: a thread owns one cc and
    // eight rows, so each cross value feeds eight FMAs (the gv reads are
    // broadcasts within the wave)
    for (int idx = t; idx < ka * (R / 8); idx += kPanelThreads) {
      const int qi = dka.div(idx), cc = idx - qi * ka, r0 = qi * 8;
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = qv[r0 + i][cc];
      for (int d = 0; d < kb; ++d) {
        const float x = cross[cc][d];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] += gv[r0 + i][d] * x;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[r0 + i][cc] = q[i] * sa_s[cc] * fold_a;
    }
    __syncthreads();
    panel_write_rows(l2 + j0 * rp, nr, rp, [&](int r, int c) -> unsigned short {
      if (c < 2 * kb) return f32_to_bf16(fv[r][c < kb ? c : c - kb]);
      c -= 2 * kb;
      if (c < 2 * ka) {
        unsigned short hi, lo;
        split_bf16(qv[r][c < ka ? c : c - ka], hi, lo);
        return c < ka ? hi : lo;
      }
      return (unsigned short)0;
    });
  }
}

// ==================================================================== GEMM
constexpr int BM = 256, BN = 256;
constexpr int BKB = 64;         // MXFP4: code bytes per row per stage (128 elements)
constexpr int ROWB = BKB + 16;  // LDS row stride (bytes), conflict-free b128 reads
constexpr int STAGE_BYTES = 2 * BM * ROWB + 2 * BM * 4;
constexpr int EPI_ROWB = 128 + 16;  // bf16 panel chunk: 64 values + pad
constexpr int NV_ROWB = 128 + 16;   // NVFP4: 64 decoded bf16 per row per stage + pad
constexpr int NV_STAGE_BYTES = 2 * BM * NV_ROWB;
constexpr int MX_LDS = 2 * STAGE_BYTES;
constexpr int NV_LDS = 2 * NV_STAGE_BYTES;
static_assert(2 * BM * EPI_ROWB <= MX_LDS && 2 * BM * EPI_ROWB <= NV_LDS, "epilogue panels must fit the main-loop LDS");
static_assert(NV_LDS <= 160 * 1024, "LDS budget of one CU");

__device__ __forceinline__ void tile_coords_of(int &tm, int &tn, int w, int nwg, int mt, int nt) {
  // XCD-aware order: consecutive dispatch ids go round-robin over the 8 XCDs;
  // regroup so each XCD walks a contiguous range of tiles, grouped 8 tile-rows
  // at a time (A and B tiles in flight on one XCD share its L2). w is the
  // tile's dispatch id among nwg; a persistent workgroup b that takes tiles
  // b, b + G, ... (G a multiple of 8) stays on the XCD of those ids.
  if ((nwg & 7) == 0) w = (w & 7) * (nwg >> 3) + (w >> 3);
  constexpr int GM = 8;
  const int group = GM * nt;
  const int g = w / group, first = g * GM;
  const int gm = min(mt - first, GM);
  const int in = w - g * group;
  tm = first + in % gm;
  tn = in / gm;
}

__device__ __forceinline__ void tile_coords(int &tm, int &tn, int mt, int nt) {
  tile_coords_of(tm, tn, blockIdx.x, gridDim.x, mt, nt);
}

// Both GEMM kernels: 256 x 256 output tile per workgroup of 512 threads,
// 8 waves in a 2 (rows) x 4 (columns) grid, each wave a 128 x 64 sub-tile of
// 4 x 2 MFMA blocks of 32 x 32 (128 accumulator registers, two waves per SIMD).
constexpr int kGemmThreads = 512;
constexpr int WM = 4, WN = 2;  // 32 x 32 blocks per wave

// acc times `scale`, plus L1[m-tile] L2[n-tile]^T (bf16, 64 panel columns at a
// time through LDS), stored as fp32.
__device__ __forceinline__ void epilogue(floatx16 (&acc)[WM][WN], float scale, uint8_t *smem, int64_t m0,
                                         int64_t n0, int64_t M, int64_t N, const unsigned short *__restrict__ l1,
                                         const unsigned short *__restrict__ l2, int rp, float *__restrict__ C,
                                         int64_t ldc) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  if (scale != 1.0f) {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] *= scale;
  }
  if (rp > 0) {
    uint8_t *L1s = smem, *L2s = smem + BM * EPI_ROWB;
    for (int c0 = 0; c0 < rp; c0 += 64) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = t + kGemmThreads * i;  // 2048 pieces of 16 bytes per panel
        const int rr = idx >> 3, piece = idx & 7;
        const int64_t ar = m0 + rr, br = n0 + rr;
        const uint4 va = ar < M ? *(const uint4 *)(l1 + ar * rp + c0 + piece * 8) : uint4{0u, 0u, 0u, 0u};
        const uint4 vb = br < N ? *(const uint4 *)(l2 + br * rp + c0 + piece * 8) : uint4{0u, 0u, 0u, 0u};
        *(uint4 *)(L1s + rr * EPI_ROWB + piece * 16) = va;
        *(uint4 *)(L2s + rr * EPI_ROWB + piece * 16) = vb;
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ushortx8 a8[WM], b8[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i)
          a8[i] = *(const ushortx8 *)(L1s + (wm * 128 + i * 32 + r32) * EPI_ROWB + ks * 32 + h * 16);
#pragma unroll
        for (int j = 0; j < WN; ++j)
          b8[j] = *(const ushortx8 *)(L2s + (wn * 64 + j * 32 + r32) * EPI_ROWB + ks * 32 + h * 16);
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) acc[i][j] = mfma32_bf16(a8[i], b8[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + r32;
      if (col >= N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * 128 + i * 32 + (q >> 2) * 8 + h * 4 + (q & 3);
        if (row < M) C[row * ldc + col] = acc[i][j][q];
      }
    }
}

// MXFP4, any K (the fallback of gemm_mx_kernel): C = Ra Rb^T (+ L1 L2^T) on
// the scaled FP4 MFMA, 128 contraction elements per LDS stage. Global loads run two stages ahead through registers
// (slot s % 2 holds stage s while it is in flight) and LDS is double
// buffered, so each load has two stages of MFMA work to land; one barrier
// per stage. Thread t stages two 16-byte pieces of A and of B per stage and
// one scale word (rows 0..255 of A for t < 256, of B above).
template <int SLOT>
__device__ __forceinline__ void mx_load(uint4 (&ga)[2][2], uint4 (&gb)[2][2], uint32_t (&gs)[2], int st,
                                        const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
                                        const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs, int64_t m0,
                                        int64_t n0, int64_t M, int64_t N, int64_t T, int64_t nb, bool scale_words) {
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)st * 128;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (t >> 2) + 128 * i, piece = t & 3;
    const int64_t e = k0 + piece * 32;
    const int64_t ar = m0 + rr, br = n0 + rr;
    ga[SLOT][i] = (ar < M && e < T) ? *(const uint4 *)(ac + ar * (T / 2) + e / 2) : uint4{0u, 0u, 0u, 0u};
    gb[SLOT][i] = (br < N && e < T) ? *(const uint4 *)(bc + br * (T / 2) + e / 2) : uint4{0u, 0u, 0u, 0u};
  }
  // four scale bytes (blocks k0/32 .. +3) of one row of one operand
  const bool isb = t >= BM;
  const int64_t row = (isb ? n0 : m0) + (t & (BM - 1));
  const bool ok = row < (isb ? N : M);
  const uint8_t *sc = (isb ? bs : as) + row * nb;
  const int64_t b0 = k0 / 32;
  if (scale_words) {  // T % 128 == 0: the four bytes are one aligned word
    gs[SLOT] = ok ? *(const uint32_t *)(sc + b0) : 0x7F7F7F7Fu;
  } else {
    uint32_t w = 0x7F7F7F7Fu;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ok && b0 + q < nb) w = (w & ~(0xFFu << (8 * q))) | ((uint32_t)sc[b0 + q] << (8 * q));
    gs[SLOT] = w;
  }
}

template <int SLOT>
__device__ __forceinline__ void mx_store(const uint4 (&ga)[2][2], const uint4 (&gb)[2][2], const uint32_t (&gs)[2],
                                         uint8_t *base) {
  const int t = threadIdx.x;
  uint8_t *A_ = base, *B_ = base + BM * ROWB;
  uint32_t *S_ = (uint32_t *)(base + 2 * BM * ROWB);  // A scale words then B scale words
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = (t >> 2) + 128 * i, piece = t & 3;
    *(uint4 *)(A_ + rr * ROWB + piece * 16) = ga[SLOT][i];
    *(uint4 *)(B_ + rr * ROWB + piece * 16) = gb[SLOT][i];
  }
  S_[t] = gs[SLOT];
}

__device__ __forceinline__ void mx_compute(floatx16 (&acc)[WM][WN], const uint8_t *base, int wm, int wn, int r32,
                                           int h) {
  const uint8_t *A_ = base, *B_ = base + BM * ROWB;
  const uint8_t *SA = base + 2 * BM * ROWB, *SB = SA + BM * 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint4 af[WM], bf[WN];
    int sa[WM], sb[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      const int rr = wm * 128 + i * 32 + r32;
      af[i] = *(const uint4 *)(A_ + rr * ROWB + h * 32 + ks * 16);
      sa[i] = SA[rr * 4 + h * 2 + ks];
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int rr = wn * 64 + j * 32 + r32;
      bf[j] = *(const uint4 *)(B_ + rr * ROWB + h * 32 + ks * 16);
      sb[j] = SB[rr * 4 + h * 2 + ks];
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = mfma_fp4(af[i], bf[j], sa[i], sb[j], acc[i][j]);
  }
}

__global__ void __launch_bounds__(kGemmThreads, 1)
    gemm_mx8_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t M,
                   const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs, int64_t N, int64_t T,
                   const unsigned short *__restrict__ l1, const unsigned short *__restrict__ l2, int rp,
                   float *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[MX_LDS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  tile_coords(tm, tn, (int)cdiv(M, BM), (int)cdiv(N, BN));
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nb = T / 32;
  const int nst = (int)cdiv(T, 128);
  const bool words = (T % 128) == 0;

  floatx16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  uint4 ga[2][2], gb[2][2];
  uint32_t gs[2];
  mx_load<0>(ga, gb, gs, 0, ac, as, bc, bs, m0, n0, M, N, T, nb, words);
  if (nst > 1) mx_load<1>(ga, gb, gs, 1, ac, as, bc, bs, m0, n0, M, N, T, nb, words);
  mx_store<0>(ga, gb, gs, smem);
  __syncthreads();
  // stage st: its data is in LDS buffer st % 2; stage st + 1 is in flight in
  // register slot (st + 1) % 2; stage st + 2 is issued into slot st % 2
  for (int st = 0; st < nst; st += 2) {
    if (st + 2 < nst) mx_load<0>(ga, gb, gs, st + 2, ac, as, bc, bs, m0, n0, M, N, T, nb, words);
    mx_compute(acc, smem, wm, wn, r32, h);
    if (st + 1 < nst) mx_store<1>(ga, gb, gs, smem + STAGE_BYTES);
    __syncthreads();
    if (st + 1 >= nst) break;
    if (st + 3 < nst) mx_load<1>(ga, gb, gs, st + 3, ac, as, bc, bs, m0, n0, M, N, T, nb, words);
    mx_compute(acc, smem + STAGE_BYTES, wm, wn, r32, h);
    if (st + 2 < nst) mx_store<0>(ga, gb, gs, smem);
    __syncthreads();
  }
  epilogue(acc, 1.0f, smem, m0, n0, M, N, l1, l2, rp, C, ldc);
}

constexpr int kMxThreads = 256;
constexpr int MXW = 4;  // 32 x 32 blocks per wave along each dimension


// The accumulators of gemm_mx_kernel stored as fp32 straight from the MFMA
// layout: lane (r32, h) of block (i, j) holds column r32 at rows
// 8 (q / 4) + 4 h + q % 4, so one store instruction writes two whole
// 128-byte row pieces (lanes 0-31 one row, 32-63 the row four below). The
// stores take their data from the accumulator registers themselves (inline
// asm with an AGPR operand; the compiler would first copy all 256 values to
// VGPRs), the four blocks of a row as immediate offsets from one address.
// Results of the last MFMAs are read only after 24 wait states.
__device__ __forceinline__ void store4_nt(float *p, float v0, float v1, float v2, float v3) {
  __asm__ volatile(
      "global_store_dword %0, %1, off nt\n\t"
      "global_store_dword %0, %2, off offset:128 nt\n\t"
      "global_store_dword %0, %3, off offset:256 nt\n\t"
      "global_store_dword %0, %4, off offset:384 nt"
      :
      : "v"(p), "a"(v0), "a"(v1), "a"(v2), "a"(v3)
      : "memory");
}
__device__ __forceinline__ void store1_nt(float *p, float v) {
  __asm__ volatile("global_store_dword %0, %1, off nt" : : "v"(p), "a"(v) : "memory");
}

__device__ __forceinline__ void store_acc_mx4(const floatx16 (&acc)[MXW][MXW], int64_t m0, int64_t n0, int64_t M,
                                              int64_t N, float *__restrict__ C, int64_t ldc) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = wm * 128 + h * 4, lc = wn * 128 + r32;  // the lane's row and column in the tile
  float *base = C + (m0 + lr) * ldc + n0 + lc;
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if (m0 + BM <= M && n0 + BN <= N) {
#pragma unroll
    for (int i = 0; i < MXW; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        float *p = base + (int64_t)(i * 32 + (q >> 2) * 8 + (q & 3)) * ldc;
        store4_nt(p, acc[i][0][q], acc[i][1][q], acc[i][2][q], acc[i][3][q]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < MXW; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int dr = i * 32 + (q >> 2) * 8 + (q & 3);
        float *p = base + (int64_t)dr * ldc;
        if (m0 + lr + dr < M) {
#pragma unroll
          for (int j = 0; j < MXW; ++j)
            if (n0 + lc + j * 32 < N) store1_nt(p + j * 32, acc[i][j][q]);
        }
      }
  }
}

// MXFP4 main kernel (K a multiple of 512): C = Ra Rb^T (+ L1 L2^T) on the
// scaled FP4 MFMA. Four waves, one per SIMD, each a 128 x 128 sub-tile (4 x 4
// MFMA blocks of 32 x 32; 256 accumulators, kept in AGPRs). Operands go
// straight from global memory to LDS (buffer loads with the LDS destination,
// 16 bytes per lane: the operand base in a buffer resource, a fixed 32-bit
// offset per lane, the stage's offset in a scalar register, so a load costs
// no vector address arithmetic; the wave index is made uniform so each LDS
// destination is a scalar)
// into a ring of four stages of 128 contraction elements (A and B codes, 256
// rows x 64 bytes each, 16-byte units XOR-swizzled by row so the fragment
// reads are conflict free: unit u of row r sits at r * 4 + (u ^ ((r / 4) & 3))),
// issued three stages ahead. The block scales of four stages (16 bytes per row
// and operand) are loaded together into a double buffer, one group ahead, so
// a row's scales cost one request per four stages. Each wave waits on its own
// load counter for the stage it needs, then a barrier; a second barrier after
// the stage's MFMAs frees its buffer. The LDS reads of the ring are done in
// asm blocks that wait for their own data, so the compiler never has to order
// them against the asynchronous loads; their outputs are early-clobber, so no
// output register doubles as an address of a later read in the same block.
// The correction L1 L2^T continues the same pipeline: after the last FP4
// stage the ring carries rp / 32 stages of 32 bf16 panel columns (64 bytes
// per row, the same swizzle), consumed by bf16 32x32x16 MFMAs, so its loads
// overlap the end of the main product instead of following it.
constexpr int kDmaStages = 4;
constexpr unsigned kMxMaxGrid = 256;  // persistent grid: one workgroup per CU (the LDS ring allows one), each
                                      // taking every 256th tile (1-3 % faster than one workgroup per tile)
constexpr int DMA_CODE_BYTES = BM * 64;            // one operand's codes per stage
constexpr int DMA_STAGE = 2 * DMA_CODE_BYTES;      // A then B
constexpr int DMA_SCALE_GROUP = 2 * BM * 16;       // A then B scales of four stages
constexpr int DMA_SCALE_BASE = kDmaStages * DMA_STAGE;
constexpr int DMA_LDS = DMA_SCALE_BASE + 2 * DMA_SCALE_GROUP;
static_assert(DMA_LDS <= 160 * 1024, "LDS budget of one CU");
static_assert(2 * BM * EPI_ROWB <= DMA_LDS, "epilogue panels must fit the main-loop LDS");

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void *)p);
}

// 16 bytes per lane from a buffer (base in the resource, voffset per lane,
// soffset uniform) straight into LDS at lds_wave_base + lane * 16
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                          void *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                         void *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 4, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding)
#define METIS_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ intx8 fp4x32v(const u32x4 v) { return intx8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0}; }

__device__ __forceinline__ floatx16 mfma_fp4_ks(const u32x4 a, const u32x4 b, int sa, int sb, floatx16 c, int ks) {
  // the scale byte is picked by opsel = ks from a word pre-shifted per lane
  return ks == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4x32v(a), fp4x32v(b), c, 4, 4, 0, sa, 0, sb)
                 : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4x32v(a), fp4x32v(b), c, 4, 4, 1, sa, 1, sb);
}

// s_waitcnt with the vector-memory count limited and every LDS read done
#define METIS_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (((n) >> 4) << 14))
// s_waitcnt for every LDS access only
#define METIS_WAIT_LDS0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14))

__global__ void __launch_bounds__(kMxThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
    gemm_mx_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t M,
                   const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs, int64_t N, int64_t T,
                   const unsigned short *__restrict__ l1, const unsigned short *__restrict__ l2, int rp,
                   float *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DMA_LDS];
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int mtiles = (int)cdiv(M, BM), ntiles_n = (int)cdiv(N, BN), ntiles = mtiles * ntiles_n;
  // buffer resources of the operands (byte ranges below 2^31 by the host's check)
  const __amdgpu_buffer_rsrc_t rA = raw_rsrc(ac, (uint32_t)(M * (T / 2))), rB = raw_rsrc(bc, (uint32_t)(N * (T / 2)));
  const __amdgpu_buffer_rsrc_t rSA = raw_rsrc(as, (uint32_t)(M * (T / 32))), rSB = raw_rsrc(bs, (uint32_t)(N * (T / 32)));
  const __amdgpu_buffer_rsrc_t rL1 = raw_rsrc(l1, (uint32_t)(M * rp * 2)), rL2 = raw_rsrc(l2, (uint32_t)(N * rp * 2));
  const int64_t nb = T / 32;
  const int nst = (int)(T / 128);
  // correction stages: 32 bf16 panel columns (64 bytes per row) of L1 rows
  // m0.. and L2 rows n0.., in the same swizzled ring layout as the codes
  const int ncs = rp / 32, ntot = nst + ncs;
  const int rA0 = wm * 128 + r32, rB0 = wn * 128 + r32;
  const int fA = (rA0 >> 2) & 3, fB = (rB0 >> 2) & 3;
  // persistent: workgroup b takes tiles b, b + gridDim.x, ... The stages of
  // its tiles form one stream through the ring: stage st of a tile sits in
  // buffer (ring0 + st) % 4 and its scale group g in (grp0 + g) % 2, so when
  // a next tile follows (and has at least eight stages) the last four steps
  // of a tile load the next tile's first four stages, and the next tile
  // starts on a full ring (pf_in) with its first stages already landed.
  int ring0 = 0, grp0 = 0;
  bool pf_in = false;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tm, tn;
    tile_coords_of(tm, tn, tile, ntiles, mtiles, ntiles_n);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const bool pf_out = tile + (int)gridDim.x < ntiles && nst >= 8;
    int64_t m0n = 0, n0n = 0;
    if (pf_out) {
      int tmn, tnn;
      tile_coords_of(tmn, tnn, tile + (int)gridDim.x, ntiles, mtiles, ntiles_n);
      m0n = (int64_t)tmn * BM;
      n0n = (int64_t)tnn * BN;
    }

    // per-lane load offsets (bytes, below 2^31 by the host's check): code unit
    // of row r = q / 4 of this wave's blocks, and the scale word of row
    // 64 wave + lane. Rows past M or N read the last row instead: their
    // products only reach rows and columns of C that are not stored.
    uint32_t offA[4], offB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 64 * (4 * wave + i) + lane, r = q >> 2, u = (q & 3) ^ ((r >> 2) & 3);
      offA[i] = (uint32_t)(min(m0 + r, M - 1) * (T / 2) + u * 16);
      offB[i] = (uint32_t)(min(n0 + r, N - 1) * (T / 2) + u * 16);
    }
    const int rs = 64 * wave + lane;
    const uint32_t offSA = (uint32_t)(min(m0 + rs, M - 1) * nb), offSB = (uint32_t)(min(n0 + rs, N - 1) * nb);

    auto issue_main = [&](int st) {  // eight loads per wave: codes of FP4 stage st
      uint8_t *sbuf = smem + ((st + ring0) & (kDmaStages - 1)) * DMA_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        buf_dma16(rA, offA[i], (uint32_t)st * 64, sbuf + (4 * wave + i) * 1024);
        buf_dma16(rB, offB[i], (uint32_t)st * 64, sbuf + DMA_CODE_BYTES + (4 * wave + i) * 1024);
      }
    };
    uint32_t offL1[4], offL2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 64 * (4 * wave + i) + lane, r = q >> 2, u = (q & 3) ^ ((r >> 2) & 3);
      offL1[i] = (uint32_t)(min(m0 + r, M - 1) * rp * 2 + u * 16);
      offL2[i] = (uint32_t)(min(n0 + r, N - 1) * rp * 2 + u * 16);
    }
    auto issue_corr = [&](int st) {  // eight loads per wave: panel columns of correction stage st
      uint8_t *sbuf = smem + ((st + ring0) & (kDmaStages - 1)) * DMA_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        buf_dma16(rL1, offL1[i], (uint32_t)(st - nst) * 64, sbuf + (4 * wave + i) * 1024);
        buf_dma16(rL2, offL2[i], (uint32_t)(st - nst) * 64, sbuf + DMA_CODE_BYTES + (4 * wave + i) * 1024);
      }
    };
    auto issue = [&](int st) {
      if (st < nst) issue_main(st);
      else issue_corr(st);
    };
    auto issue_scales = [&](int g) {  // two loads per wave: scales of stages 4 g .. 4 g + 3
      uint8_t *sg = smem + DMA_SCALE_BASE + ((g + grp0) & 1) * DMA_SCALE_GROUP;
      buf_dma16(rSA, offSA, (uint32_t)g * 16, sg + wave * 1024);
      buf_dma16(rSB, offSB, (uint32_t)g * 16, sg + BM * 16 + wave * 1024);
    };
    // stage j < 4 of the next tile (FP4: nst >= 8), its scale group 0 first,
    // into the buffers that follow this tile's last stage in the ring
    auto issue_next = [&](int j) {
      uint8_t *sbuf = smem + ((ring0 + ntot + j) & (kDmaStages - 1)) * DMA_STAGE;
      if (j == 0) {
        uint8_t *sg = smem + DMA_SCALE_BASE + ((grp0 + nst / 4) & 1) * DMA_SCALE_GROUP;
        buf_dma16(rSA, (uint32_t)(min(m0n + rs, M - 1) * nb), 0u, sg + wave * 1024);
        buf_dma16(rSB, (uint32_t)(min(n0n + rs, N - 1) * nb), 0u, sg + BM * 16 + wave * 1024);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = 64 * (4 * wave + i) + lane, r = q >> 2, u = (q & 3) ^ ((r >> 2) & 3);
        buf_dma16(rA, (uint32_t)(min(m0n + r, M - 1) * (T / 2) + u * 16), (uint32_t)j * 64,
                  sbuf + (4 * wave + i) * 1024);
        buf_dma16(rB, (uint32_t)(min(n0n + r, N - 1) * (T / 2) + u * 16), (uint32_t)j * 64,
                  sbuf + DMA_CODE_BYTES + (4 * wave + i) * 1024);
      }
    };
    // Wait until the codes of stage s (and the scales of its group, issued
    // before them) have landed: at most the 8 loads of each later stage
    // issued so far (s + 1 .. min(s + 2, ntot - 1)) may still be pending. A
    // scale group issued among them only makes the wait stricter than needed.
    // Every LDS read of the wave is also complete afterwards.
    auto wait_stage = [&](int s) {
      const int d = min(s + 2, ntot - 1) - s;
      if (d >= 2) METIS_WAIT_VMCNT_LDS(16);
      else if (d == 1) METIS_WAIT_VMCNT_LDS(8);
      else METIS_WAIT_VMCNT_LDS(0);
    };
    // fragments of half ks of stage st: 16-byte unit 2 h + ks of the row
    // (FP4: lane half h takes K 32 h .. of the 64 the MFMA covers) or 2 ks + h
    // (bf16 panels: 8 consecutive columns), and for FP4 half 0 the stage's
    // block-scale word of each row (its bytes 2 h + ks serve half ks)
    auto load_frags_k = [&](int st, int ks, auto corr, u32x4 (&af)[MXW], u32x4 (&bf)[MXW], int (&sa)[MXW],
                            int (&sb)[MXW]) {
      constexpr bool CORR = decltype(corr)::value;
      const uint8_t *base = smem + ((st + ring0) & (kDmaStages - 1)) * DMA_STAGE;
      const int un = CORR ? 2 * ks + h : 2 * h + ks;
      const uint8_t *pa = base + rA0 * 64 + ((un ^ fA) << 4);
      const uint8_t *pb = base + DMA_CODE_BYTES + rB0 * 64 + ((un ^ fB) << 4);
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        af[i] = *(const u32x4 *)(pa + i * 2048);
        bf[i] = *(const u32x4 *)(pb + i * 2048);
      }
      if (!CORR && ks == 0) {
        const uint8_t *sbase = smem + DMA_SCALE_BASE + ((st / 4 + grp0) & 1) * DMA_SCALE_GROUP + (st % 4) * 4;
#pragma unroll
        for (int i = 0; i < MXW; ++i) {
          sa[i] = *(const int *)(sbase + (rA0 + 32 * i) * 16);
          sb[i] = *(const int *)(sbase + BM * 16 + (rB0 + 32 * i) * 16);
        }
      }
    };
    auto load_frags = [&](int st, int ks, u32x4 (&af)[MXW], u32x4 (&bf)[MXW], int (&sa)[MXW], int (&sb)[MXW]) {
      if (st < nst) load_frags_k(st, ks, std::false_type{}, af, bf, sa, sb);
      else load_frags_k(st, ks, std::true_type{}, af, bf, sa, sb);
    };

    floatx16 acc[MXW][MXW];
#pragma unroll
    for (int i = 0; i < MXW; ++i)
#pragma unroll
      for (int j = 0; j < MXW; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    auto mfmas = [&](int ks, auto corr, const u32x4 (&af)[MXW], const u32x4 (&bf)[MXW], const int (&sa)[MXW],
                     const int (&sb)[MXW]) {
      if constexpr (!decltype(corr)::value) {
        int xa[MXW], xb[MXW];  // scale words shifted so opsel = ks picks byte 2 h + ks
#pragma unroll
        for (int i = 0; i < MXW; ++i) {
          xa[i] = (int)((uint32_t)sa[i] >> (16 * h));
          xb[i] = (int)((uint32_t)sb[i] >> (16 * h));
        }
#pragma unroll
        for (int i = 0; i < MXW; ++i)
#pragma unroll
          for (int j = 0; j < MXW; ++j) acc[i][j] = mfma_fp4_ks(af[i], bf[j], xa[i], xb[j], acc[i][j], ks);
      } else {
#pragma unroll
        for (int i = 0; i < MXW; ++i)
#pragma unroll
          for (int j = 0; j < MXW; ++j)
            acc[i][j] = mfma32_bf16(__builtin_bit_cast(ushortx8, af[i]), __builtin_bit_cast(ushortx8, bf[j]), acc[i][j]);
      }
    };

    // Pipeline: half 1 of stage st is read while the MFMAs of half 0 run; a
    // barrier (stage st + 1 landed, every read of stage st done) frees buffer
    // st % 4 for stage st + 4; half 0 of stage st + 1 is read while the MFMAs
    // of half 1 run. Prologue: scales(0), codes(0 .. 2), then after the first
    // barrier codes(3) and scales(1); iteration st issues codes(st + 4) and,
    // right after codes(4 g - 1), scales(g).
    u32x4 a0f[MXW], b0f[MXW], a1f[MXW], b1f[MXW];
    int s0a[MXW], s0b[MXW], s1a[MXW], s1b[MXW];
    if (pf_in) {
      // stages 0 .. 3 landed before the previous tile's stores (each wave
      // waited for its own loads; the barrier covers the others')
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    } else {
      issue_scales(0);
      issue(0);
      if (ntot > 1) issue(1);
      if (ntot > 2) issue(2);
      wait_stage(0);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      if (ntot > 3) issue(3);
    }
    if (4 < nst) issue_scales(1);
    load_frags(0, 0, a0f, b0f, s0a, s0b);
    // One pipeline step; the FP4 stages and the bf16 correction stages run
    // in loops of their own so each MFMA kind keeps the accumulators in
    // place. In a steady step the kinds of stage st (corr), of stage st + 1
    // (whose half 0 is read, nextc) and of stage st + 4 (whose DMA is issued,
    // dmac) are known at compile time and stages st + 1 .. st + 4 exist, so
    // the DMA issue and the fragment reads share one basic block with the
    // MFMAs of half 1 and can be spread between them; a scale group, when
    // due, follows the MFMAs. (Scheduling barriers keep the parts in order:
    // the compiler would otherwise gather both MFMA halves behind one wait
    // for all reads.)
    auto step = [&](int st, auto corr, auto steady, auto nextc, auto dmac, auto landed) {
      constexpr bool STEADY = decltype(steady)::value;
      // half 0 (read during the previous MFMA half) is complete before half
      // 1's reads are issued, so the MFMAs below wait for nothing
      __asm__ volatile("" : "+v"(a0f[0]), "+v"(a0f[1]), "+v"(a0f[2]), "+v"(a0f[3]), "+v"(b0f[0]), "+v"(b0f[1]),
                       "+v"(b0f[2]), "+v"(b0f[3]), "+v"(s0a[0]), "+v"(s0a[1]), "+v"(s0a[2]), "+v"(s0a[3]),
                       "+v"(s0b[0]), "+v"(s0b[1]), "+v"(s0b[2]), "+v"(s0b[3]));
      load_frags_k(st, 1, corr, a1f, b1f, s1a, s1b);
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        s1a[i] = s0a[i];
        s1b[i] = s0b[i];
      }
      mfmas(0, corr, a0f, b0f, s0a, s0b);
      // half 1's reads go out between the first MFMAs of half 0
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      // the MFMAs are pure, so the optimizer may move them across the
      // barrier; empty asm statements that take the accumulators here and
      // hand out half 1's fragments after the barrier pin them in place
      __asm__ volatile("" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                       "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
                       "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
                       "+a"(acc[3][3]));
      __builtin_amdgcn_sched_barrier(0);
      __asm__ volatile("" ::: "memory");
      if constexpr (decltype(landed)::value) {
        METIS_WAIT_LDS0();  // stage st + 1 landed before the previous tile's stores
      } else if constexpr (STEADY) {
        METIS_WAIT_VMCNT_LDS(16);
      } else if (pf_out) {
        // the stream goes on into the next tile: at most the two stages after
        // st + 1 (and a scale group) are pending
        if (st + 1 < ntot) METIS_WAIT_VMCNT_LDS(16);
        else METIS_WAIT_LDS0();
      } else {
        if (st + 1 < ntot) wait_stage(st + 1);
        else METIS_WAIT_VMCNT_LDS(0);
      }
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      __asm__ volatile("" : "+v"(a1f[0]), "+v"(a1f[1]), "+v"(a1f[2]), "+v"(a1f[3]), "+v"(b1f[0]), "+v"(b1f[1]),
                       "+v"(b1f[2]), "+v"(b1f[3]));
      if constexpr (STEADY) {
        if constexpr (decltype(dmac)::value) issue_corr(st + 4);
        else issue_main(st + 4);
        load_frags_k(st + 1, 0, nextc, a0f, b0f, s0a, s0b);
      } else {
        if (st + 4 < ntot) issue(st + 4);
        else if (pf_out) issue_next(st + 4 - ntot);
        if ((st + 1) % 4 == 0 && 4 * ((st + 1) / 4 + 1) < nst) issue_scales((st + 1) / 4 + 1);
        if (st + 1 < ntot) load_frags(st + 1, 0, a0f, b0f, s0a, s0b);
      }
      mfmas(1, corr, a1f, b1f, s1a, s1b);
      // the DMA of stage st + 4 and the reads of half 0 of stage st + 1 go
      // out between the MFMAs of half 1
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 1);  // two global loads (to LDS)
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (STEADY && !decltype(corr)::value) {
        if ((st + 1) % 4 == 0 && 4 * ((st + 1) / 4 + 1) < nst) issue_scales((st + 1) / 4 + 1);
      }
    };
    using F = std::false_type;
    using Tt = std::true_type;
    int st = 0;
    if (pf_in) {
      // nst >= 8: the first group is steady; stages 1 .. 3 need no wait
      step(0, F{}, Tt{}, F{}, F{}, Tt{});
      step(1, F{}, Tt{}, F{}, F{}, Tt{});
      step(2, F{}, Tt{}, F{}, F{}, Tt{});
      step(3, F{}, Tt{}, F{}, F{}, F{});
      st = 4;
    }
    // FP4 stages whose next four stages are FP4 stages too, four per group
    for (; st + 7 < nst; st += 4) {
      step(st, F{}, Tt{}, F{}, F{}, F{});
      step(st + 1, F{}, Tt{}, F{}, F{}, F{});
      step(st + 2, F{}, Tt{}, F{}, F{}, F{});
      step(st + 3, F{}, Tt{}, F{}, F{}, F{});
    }
    if (ncs >= 4 && st + 4 == nst) {
      // the last four FP4 stages issue the first correction stages
      step(st, F{}, Tt{}, F{}, Tt{}, F{});
      step(st + 1, F{}, Tt{}, F{}, Tt{}, F{});
      step(st + 2, F{}, Tt{}, F{}, Tt{}, F{});
      step(st + 3, F{}, Tt{}, Tt{}, Tt{}, F{});
      st += 4;
    }
    for (; st < nst; ++st) step(st, F{}, F{}, F{}, F{}, F{});
    for (; st + 4 < ntot; ++st) step(st, Tt{}, Tt{}, Tt{}, Tt{}, F{});
    for (; st < ntot; ++st) step(st, Tt{}, F{}, F{}, F{}, F{});
    // every LDS read of the tile finished before the last barrier. With a
    // next tile in the stream, its stages 0 .. 3 (and scale group 0) are
    // waited for before the stores, since a wait issued after them would also
    // wait for the stores. Otherwise the next tile's first loads refill the
    // ring while these stores drain.
    if (pf_out) METIS_WAIT_VMCNT_LDS(0);
    store_acc_mx4(acc, m0, n0, M, N, C, ldc);
    ring0 = (ring0 + ntot) & (kDmaStages - 1);
    grp0 = (grp0 + nst / 4) & 1;
    pf_in = pf_out;
  }
}

// NVFP4 main kernel on the same ring (K a multiple of 128): C = ts_a ts_b
// (Ra Rb^T) + L1 L2^T. Four waves, one per SIMD, each a 128 x 128 sub-tile
// (4 x 4 blocks of 32 x 32, 256 accumulators). A stage of 128 contraction
// elements holds the codes of A and B (256 rows x 64 bytes each, the swizzled
// 16-byte units of the MXFP4 kernel) and their E4M3 block scales (8 bytes per
// row), all loaded straight to LDS; stage st + 4 is requested once every
// wave has read stage st, half-way through it. Lane (r, h) of a wave
// reads the 64 codes of its row's half h (two units) and its half's four
// scale bytes; step s of the stage's eight fp16 32x32x16 MFMA steps takes the
// lane's codes 8 s .. 8 s + 7, decoded exactly to fp16 with their block's
// scale (the hardware FP4 conversion and one packed multiply, as in the
// skinny NVFP4 products). A and B lanes take the same contraction elements
// in every step, so the products pair up; the contraction order differs from
// the natural one only in how the fp32 sums are grouped. After the last FP4
// stage the accumulators take the product of the two tensor scales; the bf16
// correction stages follow through the same ring.
constexpr int NVD_SC_BYTES = BM * 8;  // one operand's E4M3 scales per stage
constexpr int NVD_STAGE = 2 * DMA_CODE_BYTES + 2 * NVD_SC_BYTES;
constexpr int NVD_LDS = kDmaStages * NVD_STAGE;
static_assert(NVD_LDS <= 160 * 1024, "LDS budget of one CU");

__global__ void __launch_bounds__(kMxThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
    gemm_nvd_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, const float *__restrict__ ats,
                    int64_t M, const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs,
                    const float *__restrict__ bts, int64_t N, int64_t T, const unsigned short *__restrict__ l1,
                    const unsigned short *__restrict__ l2, int rp, float *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NVD_LDS];
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int mtiles = (int)cdiv(M, BM), ntiles_n = (int)cdiv(N, BN), ntiles = mtiles * ntiles_n;
  const int64_t nbs = T / 16;  // scale bytes per row
  // buffer resources (byte ranges below 2^31 by the host's check)
  const __amdgpu_buffer_rsrc_t rA = raw_rsrc(ac, (uint32_t)(M * (T / 2))), rB = raw_rsrc(bc, (uint32_t)(N * (T / 2)));
  const __amdgpu_buffer_rsrc_t rSA = raw_rsrc(as, (uint32_t)(M * nbs)), rSB = raw_rsrc(bs, (uint32_t)(N * nbs));
  const __amdgpu_buffer_rsrc_t rL1 = raw_rsrc(l1, (uint32_t)(M * rp * 2)), rL2 = raw_rsrc(l2, (uint32_t)(N * rp * 2));
  const int nst = (int)(T / 128), ncs = rp / 32, ntot = nst + ncs;
  const float tscale = ats[0] * bts[0] * 65536.0f;
  const int rA0 = wm * 128 + r32, rB0 = wn * 128 + r32;
  const int fA = (rA0 >> 2) & 3, fB = (rB0 >> 2) & 3;  // the same for rows + 32 i
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    int tm, tn;
    tile_coords_of(tm, tn, tile, ntiles, mtiles, ntiles_n);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    // per-lane load offsets (rows past M or N read the last row: their
    // products reach only rows and columns of C that are not stored)
    uint32_t offA[4], offB[4], offL1[4], offL2[4], offSA[2], offSB[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 64 * (4 * wave + i) + lane, r = q >> 2, u = (q & 3) ^ ((r >> 2) & 3);
      const int64_t ra = min(m0 + r, M - 1), rb = min(n0 + r, N - 1);
      offA[i] = (uint32_t)(ra * (T / 2) + u * 16);
      offB[i] = (uint32_t)(rb * (T / 2) + u * 16);
      offL1[i] = (uint32_t)(ra * rp * 2 + u * 16);
      offL2[i] = (uint32_t)(rb * rp * 2 + u * 16);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // 4-byte piece q of the stage's scales: row q / 2, half q % 2
      const int q = 128 * wave + 64 * u + lane, r = q >> 1;
      offSA[u] = (uint32_t)(min(m0 + r, M - 1) * nbs + (q & 1) * 4);
      offSB[u] = (uint32_t)(min(n0 + r, N - 1) * nbs + (q & 1) * 4);
    }
    auto issue_main = [&](int st) {  // twelve loads per wave: codes and scales of FP4 stage st
      uint8_t *sbuf = smem + (st % kDmaStages) * NVD_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        buf_dma16(rA, offA[i], (uint32_t)st * 64, sbuf + (4 * wave + i) * 1024);
        buf_dma16(rB, offB[i], (uint32_t)st * 64, sbuf + DMA_CODE_BYTES + (4 * wave + i) * 1024);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        buf_dma4(rSA, offSA[u], (uint32_t)st * 8, sbuf + 2 * DMA_CODE_BYTES + (128 * wave + 64 * u) * 4);
        buf_dma4(rSB, offSB[u], (uint32_t)st * 8, sbuf + 2 * DMA_CODE_BYTES + NVD_SC_BYTES + (128 * wave + 64 * u) * 4);
      }
    };
    auto issue_corr = [&](int st) {  // eight loads per wave: 32 bf16 panel columns
      uint8_t *sbuf = smem + (st % kDmaStages) * NVD_STAGE;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        buf_dma16(rL1, offL1[i], (uint32_t)(st - nst) * 64, sbuf + (4 * wave + i) * 1024);
        buf_dma16(rL2, offL2[i], (uint32_t)(st - nst) * 64, sbuf + DMA_CODE_BYTES + (4 * wave + i) * 1024);
      }
    };
    auto issue = [&](int st) {
      if (st < nst) issue_main(st);
      else if (st < ntot) issue_corr(st);
    };
    // stage s has landed once at most the loads of the later stages issued
    // so far (s + 1, s + 2) are pending; every LDS read of the wave is done too
    auto wait_stage = [&](int s) {
      int n = 0;
      for (int k = s + 1; k <= min(s + 2, ntot - 1); ++k) n += k < nst ? 12 : 8;
      switch (n) {
        case 24: METIS_WAIT_VMCNT_LDS(24); break;
        case 20: METIS_WAIT_VMCNT_LDS(20); break;
        case 16: METIS_WAIT_VMCNT_LDS(16); break;
        case 12: METIS_WAIT_VMCNT_LDS(12); break;
        case 8: METIS_WAIT_VMCNT_LDS(8); break;
        default: METIS_WAIT_VMCNT_LDS(0); break;
      }
    };
    floatx16 acc[MXW][MXW];
    auto pin_acc = [&] {
      __asm__ volatile("" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                       "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
                       "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
                       "+a"(acc[3][3]));
    };
#pragma unroll
    for (int i = 0; i < MXW; ++i)
#pragma unroll
      for (int j = 0; j < MXW; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    // A stage is consumed in two halves of four 32x32x16 steps: half v uses
    // unit 2 h + v of the lane's row (steps 4 v .. 4 v + 3) and scale bytes
    // 2 v, 2 v + 1. Half 1 of stage st is read while the MFMAs of half 0 run;
    // then one barrier (stage st + 1 landed, every read of stage st done)
    // frees buffer st % 4 for stage st + 4, and half 0 of stage st + 1 is
    // read while the MFMAs of half 1 run. Each step's MFMAs run while the
    // next step's operands are decoded.
    u32x4 c0a[MXW], c0b[MXW], c1a[MXW], c1b[MXW];
    uint32_t s0a[MXW], s0b[MXW], s1a[MXW], s1b[MXW];
    halfx8 fa0[MXW], fb0[MXW], fa1[MXW], fb1[MXW];
    auto read_half = [&](int st, int v, u32x4 (&ca)[MXW], u32x4 (&cb)[MXW]) {
      const uint8_t *base = smem + (st % kDmaStages) * NVD_STAGE;
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        ca[i] = *(const u32x4 *)(base + (rA0 + 32 * i) * 64 + (((2 * h + v) ^ fA) << 4));
        cb[i] = *(const u32x4 *)(base + DMA_CODE_BYTES + (rB0 + 32 * i) * 64 + (((2 * h + v) ^ fB) << 4));
      }
    };
    auto read_scales = [&](int st) {  // the four scale bytes of the lane's row half
      const uint8_t *base = smem + (st % kDmaStages) * NVD_STAGE + 2 * DMA_CODE_BYTES;
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        s0a[i] = *(const uint32_t *)(base + (rA0 + 32 * i) * 8 + 4 * h);
        s0b[i] = *(const uint32_t *)(base + NVD_SC_BYTES + (rB0 + 32 * i) * 8 + 4 * h);
      }
    };
    // A block scale as an fp16 pair: the E4M3 byte's sign, exponent and
    // mantissa moved into the fp16 fields give its value times 2^-8 exactly
    // (normal and subnormal E4M3 alike), so each decoded product is an exact
    // fp16 value (a multiple of 2^-18 below 11); the 2^16 the two operands
    // lose is given back with the tensor scales.
    auto scale2 = [](uint32_t word, int b) {
      const uint32_t e = (word >> (8 * b)) & 255u;
      const uint32_t f = ((e & 0x80u) << 8) | ((e & 0x7Fu) << 7);
      return __builtin_bit_cast(halfx2, f | (f << 16));
    };
    // step s of a stage: code word s % 4 of the half's unit, scale byte s / 2
    auto decode = [&](int s, const u32x4 (&ca)[MXW], const u32x4 (&cb)[MXW], const uint32_t (&sa)[MXW],
                      const uint32_t (&sb)[MXW], halfx8 (&af)[MXW], halfx8 (&bf)[MXW]) {
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        af[i] = fp4x8_to_f16(ca[i][s & 3], scale2(sa[i], s >> 1));
        bf[i] = fp4x8_to_f16(cb[i][s & 3], scale2(sb[i], s >> 1));
      }
    };
    auto mfmas16 = [&](const halfx8 (&af)[MXW], const halfx8 (&bf)[MXW]) {
#pragma unroll
      for (int i = 0; i < MXW; ++i)
#pragma unroll
        for (int j = 0; j < MXW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    };
    // the MFMAs of a step with the next step's decode spread between them
    // (and, where given, nr LDS reads or nv global loads placed first)
    auto sched = [](auto nr, auto nv) {
      constexpr int R = decltype(nr)::value, V = decltype(nv)::value;
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if constexpr (V > 0) {
          if (g < V) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load (to LDS)
        }
        if constexpr (R > 0) {
          if (g >= V && g < V + R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    using I0 = std::integral_constant<int, 0>;
    // one FP4 stage; LAST: stage st + 1 is not an FP4 stage (no half 0 to
    // read and decode ahead)
    auto fp4_stage = [&](int st, auto last) {
      constexpr bool LAST = decltype(last)::value;
      read_half(st, 1, c1a, c1b);
      decode(1, c0a, c0b, s0a, s0b, fa1, fb1);
      mfmas16(fa0, fb0);
      sched(std::integral_constant<int, 8>{}, I0{});
      decode(2, c0a, c0b, s0a, s0b, fa0, fb0);
      mfmas16(fa1, fb1);
      sched(I0{}, I0{});
      decode(3, c0a, c0b, s0a, s0b, fa1, fb1);
      mfmas16(fa0, fb0);
      sched(I0{}, I0{});
      decode(4, c1a, c1b, s0a, s0b, fa0, fb0);
      mfmas16(fa1, fb1);
      sched(I0{}, I0{});
#pragma unroll
      for (int i = 0; i < MXW; ++i) {
        s1a[i] = s0a[i];
        s1b[i] = s0b[i];
      }
      // the MFMAs are pure and could move across the barrier: empty asm
      // statements pin the accumulators before it and the decoded operands
      // of step 4 after it
      pin_acc();
      __builtin_amdgcn_sched_barrier(0);
      __asm__ volatile("" ::: "memory");
      wait_stage(st + 1);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      __asm__ volatile("" : "+v"(fa0[0]), "+v"(fa0[1]), "+v"(fa0[2]), "+v"(fa0[3]), "+v"(fb0[0]), "+v"(fb0[1]),
                       "+v"(fb0[2]), "+v"(fb0[3]));
      issue(st + 4);
      if constexpr (!LAST) {
        read_half(st + 1, 0, c0a, c0b);
        read_scales(st + 1);
      }
      decode(5, c1a, c1b, s1a, s1b, fa1, fb1);
      mfmas16(fa0, fb0);
      sched(I0{}, std::integral_constant<int, 12>{});
      decode(6, c1a, c1b, s1a, s1b, fa0, fb0);
      mfmas16(fa1, fb1);
      sched(std::integral_constant<int, LAST ? 0 : 16>{}, I0{});
      decode(7, c1a, c1b, s1a, s1b, fa1, fb1);
      mfmas16(fa0, fb0);
      sched(I0{}, I0{});
      if constexpr (!LAST) decode(0, c0a, c0b, s0a, s0b, fa0, fb0);
      mfmas16(fa1, fb1);
      sched(I0{}, I0{});
      pin_acc();
    };
    issue(0);
    issue(1);
    issue(2);
    wait_stage(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    issue(3);
    read_half(0, 0, c0a, c0b);
    read_scales(0);
    decode(0, c0a, c0b, s0a, s0b, fa0, fb0);
    int st = 0;
    for (; st + 1 < nst; ++st) fp4_stage(st, std::false_type{});
    fp4_stage(st, std::true_type{});
#pragma unroll
    for (int i = 0; i < MXW; ++i)
#pragma unroll
      for (int j = 0; j < MXW; ++j) acc[i][j] *= tscale;  // includes the 2^16 of the scale decoding
    pin_acc();
    // correction stages (stage st landed and the barrier after it passed):
    // read, wait for stage st + 1 and every read, barrier, refill, MFMAs
    for (st = nst; st < ntot; ++st) {
      read_half(st, 0, c0a, c0b);  // units 2 h and 2 h + 1: panel columns 16 h .. 16 h + 15
      read_half(st, 1, c1a, c1b);
      wait_stage(st + 1);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      issue(st + 4);
#pragma unroll
      for (int i = 0; i < MXW; ++i)
#pragma unroll
        for (int j = 0; j < MXW; ++j)
          acc[i][j] = mfma32_bf16(__builtin_bit_cast(ushortx8, c0a[i]), __builtin_bit_cast(ushortx8, c0b[j]), acc[i][j]);
#pragma unroll
      for (int i = 0; i < MXW; ++i)
#pragma unroll
        for (int j = 0; j < MXW; ++j)
          acc[i][j] = mfma32_bf16(__builtin_bit_cast(ushortx8, c1a[i]), __builtin_bit_cast(ushortx8, c1b[j]), acc[i][j]);
      pin_acc();
    }
    store_acc_mx4(acc, m0, n0, M, N, C, ldc);
  }
}

// Skinny products on the DMA path (MXFP4, T a multiple of 256): out[s]
// (rows x cols, cols <= 32 NCT) = NT(A, B) over T-chunk s. A workgroup of
// four waves takes 128 rows of A (wave w: rows 32 w ..) and all of B; a stage
// is 256 contraction elements (128 code bytes and 8 scale bytes per row).
// Codes go to LDS with 16-byte buffer loads (LDS destination), eight lanes per row, so one
// load instruction covers eight whole 128-byte row pieces (loading them in
// the MFMA's own layout, one row per lane, made the address units the
// bottleneck); slot 8 r + (u ^ (r & 7)) of a stage holds unit u of row r,
// which keeps the fragment reads free of bank conflicts. Scales follow with
// 4-byte loads, two per row. A ring of three stages is kept in flight (at
// most two column tiles: 78 KB, so two workgroups share a CU; a split has
// only four to six stages, so a workgroup is mostly waiting for its loads).
// Rows past the end read the last row: their products reach only rows or
// columns that are not stored.
constexpr int kSkRows = 128;
constexpr int kSkStages = 3;
template <int NCT>
struct SkLayout {
  static constexpr int A_CODES = 0;
  static constexpr int B_CODES = kSkRows * 128;
  static constexpr int A_SC = B_CODES + 32 * NCT * 128;
  static constexpr int B_SC = A_SC + kSkRows * 8;
  static constexpr int STAGE = B_SC + 32 * NCT * 8;
  static constexpr int LOADS = 4 + NCT + 2;  // DMA instructions per wave and stage
};

// LDS reads of one skinny stage. Scales: the two words of the lane's A row
// and of its B rows 32 j + r (rows 256 bytes apart). Codes: for K-block kk
// the 16-byte unit 2 kk + h of the lane's A row and B rows, at slot
// unit ^ (row & 7) (B rows 32 j + r share r & 7, so they are 4096 bytes
// apart). Each asm block waits for its own loads.
template <int NCT>
__device__ __forceinline__ void skinny_read_scales(uint32_t pa, uint32_t pb, uint32_t (&wa)[2], uint32_t (&wb)[NCT][2]) {
  uint2 a, b0, b1, b2;
  if constexpr (NCT == 1) {
    asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b0) : "v"(pa), "v"(pb) : "memory");
  } else if constexpr (NCT == 2) {
    asm volatile("ds_read_b64 %0, %3\n\tds_read_b64 %1, %4\n\tds_read_b64 %2, %4 offset:256\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b0), "=&v"(b1) : "v"(pa), "v"(pb) : "memory");
  } else {
    asm volatile("ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %5 offset:256\n\t"
                 "ds_read_b64 %3, %5 offset:512\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b0), "=&v"(b1), "=&v"(b2) : "v"(pa), "v"(pb) : "memory");
  }
  wa[0] = a.x; wa[1] = a.y;
  wb[0][0] = b0.x; wb[0][1] = b0.y;
  if constexpr (NCT > 1) { wb[1][0] = b1.x; wb[1][1] = b1.y; }
  if constexpr (NCT > 2) { wb[2][0] = b2.x; wb[2][1] = b2.y; }
}

template <int NCT>
__device__ __forceinline__ void skinny_read_codes(uint32_t ra, uint32_t rb, int x, int h, u32x4 (&fa)[4],
                                                  u32x4 (&fb)[4][NCT]) {
  uint32_t pa[4], pb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t off = (uint32_t)(((2 * kk + h) ^ x) << 4);
    pa[kk] = ra + off;
    pb[kk] = rb + off;
  }
  if constexpr (NCT == 1) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3]), "=&v"(fb[0][0]), "=&v"(fb[1][0]), "=&v"(fb[2][0]),
          "=&v"(fb[3][0])
        : "v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]), "v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3])
        : "memory");
  } else if constexpr (NCT == 2) {
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %1, %13\n\tds_read_b128 %2, %14\n\tds_read_b128 %3, %15\n\t"
        "ds_read_b128 %4, %16\n\tds_read_b128 %5, %16 offset:4096\n\t"
        "ds_read_b128 %6, %17\n\tds_read_b128 %7, %17 offset:4096\n\t"
        "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:4096\n\t"
        "ds_read_b128 %10, %19\n\tds_read_b128 %11, %19 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3]), "=&v"(fb[0][0]), "=&v"(fb[0][1]), "=&v"(fb[1][0]),
          "=&v"(fb[1][1]), "=&v"(fb[2][0]), "=&v"(fb[2][1]), "=&v"(fb[3][0]), "=&v"(fb[3][1])
        : "v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]), "v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %17\n\tds_read_b128 %2, %18\n\tds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %20\n\tds_read_b128 %5, %20 offset:4096\n\tds_read_b128 %6, %20 offset:8192\n\t"
        "ds_read_b128 %7, %21\n\tds_read_b128 %8, %21 offset:4096\n\tds_read_b128 %9, %21 offset:8192\n\t"
        "ds_read_b128 %10, %22\n\tds_read_b128 %11, %22 offset:4096\n\tds_read_b128 %12, %22 offset:8192\n\t"
        "ds_read_b128 %13, %23\n\tds_read_b128 %14, %23 offset:4096\n\tds_read_b128 %15, %23 offset:8192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3]), "=&v"(fb[0][0]), "=&v"(fb[0][1]), "=&v"(fb[0][2]),
          "=&v"(fb[1][0]), "=&v"(fb[1][1]), "=&v"(fb[1][2]), "=&v"(fb[2][0]), "=&v"(fb[2][1]), "=&v"(fb[2][2]),
          "=&v"(fb[3][0]), "=&v"(fb[3][1]), "=&v"(fb[3][2])
        : "v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]), "v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3])
        : "memory");
  }
}

template <int OP>
__device__ __forceinline__ floatx16 mfma_fp4_op(const uint4 a, const uint4 b, int sa, int sb, floatx16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4x32(a), fp4x32(b), c, 4, 4, OP, sa, OP, sb);
}

// The product of row block bx and contraction split by (the body of both
// skinny kernels below).
template <int NCT>
__device__ __forceinline__ void skinny_dma_block(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
                                                 int64_t rows, const uint8_t *__restrict__ bc,
                                                 const uint8_t *__restrict__ bs, int cols, int64_t T, int64_t chunk,
                                                 float *__restrict__ out, int bx, int by) {
  using L = SkLayout<NCT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSkStages * L::STAGE];
  const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, r = lane & 31, h = lane >> 5;
  const int64_t row0 = (int64_t)bx * kSkRows;
  const int64_t t_beg = (int64_t)by * chunk, t_end = std::min<int64_t>(T, t_beg + chunk);
  const int nst = (int)((t_end - t_beg) / 256);
  const int64_t nbr = T / 32;  // scale bytes per row
  // per-thread sources (byte offsets below 2^31 by the host's check)
  uint32_t offA[4], offB[NCT];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = t + 256 * i, rr = p >> 3, u = (p & 7) ^ (rr & 7);
    offA[i] = (uint32_t)(std::min<int64_t>(row0 + rr, rows - 1) * (T / 2) + u * 16);
  }
#pragma unroll
  for (int i = 0; i < NCT; ++i) {
    const int p = t + 256 * i, rr = p >> 3, u = (p & 7) ^ (rr & 7);
    offB[i] = (uint32_t)(std::min(rr, cols - 1) * (T / 2) + u * 16);
  }
  const uint32_t offSA = (uint32_t)(std::min<int64_t>(row0 + (t >> 1), rows - 1) * nbr + 4 * (t & 1));
  const int pb = t % (64 * NCT);  // waves past NCT repeat the same loads (same bytes to the same slots)
  const uint32_t offSB = (uint32_t)(std::min(pb >> 1, cols - 1) * nbr + 4 * (pb & 1));
  // buffer resources (byte ranges below 2^31 by the host's check): the loads
  // take a fixed 32-bit offset per lane and the stage's offset as a scalar
  const __amdgpu_buffer_rsrc_t rA = raw_rsrc(ac, (uint32_t)(rows * (T / 2))), rB = raw_rsrc(bc, (uint32_t)(cols * (T / 2)));
  const __amdgpu_buffer_rsrc_t rSA = raw_rsrc(as, (uint32_t)(rows * nbr)), rSB = raw_rsrc(bs, (uint32_t)(cols * nbr));
  auto issue = [&](int st) {
    uint8_t *sb = smem + (st % kSkStages) * L::STAGE;
    const int64_t k0 = t_beg + 256 * (int64_t)st;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf_dma16(rA, offA[i], (uint32_t)(k0 / 2), sb + L::A_CODES + (256 * i + 64 * wave) * 16);
#pragma unroll
    for (int i = 0; i < NCT; ++i)
      buf_dma16(rB, offB[i], (uint32_t)(k0 / 2), sb + L::B_CODES + (256 * i + 64 * wave) * 16);
    buf_dma4(rSA, offSA, (uint32_t)(k0 / 32), sb + L::A_SC + 64 * wave * 4);
    buf_dma4(rSB, offSB, (uint32_t)(k0 / 32), sb + L::B_SC + (64 * wave % (64 * NCT)) * 4);
  };
  floatx16 acc[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.0f;
  const int ra_ = 32 * wave + r;  // this lane's A row in the block
  for (int st = 0; st < kSkStages && st < nst; ++st) issue(st);
  for (int st = 0; st < nst; ++st) {
    // stage st has landed once at most the later stages' loads are pending
    // (a plain __syncthreads would also wait for every later stage)
    switch (std::min(kSkStages - 1, nst - 1 - st)) {
      case 3: METIS_WAIT_VMCNT(3 * L::LOADS); break;
      case 2: METIS_WAIT_VMCNT(2 * L::LOADS); break;
      case 1: METIS_WAIT_VMCNT(1 * L::LOADS); break;
      default: METIS_WAIT_VMCNT(0); break;
    }
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");  // the reads below stay after the barrier
    // the stage's reads in asm blocks that wait for their own data (the
    // compiler would otherwise order them after every DMA still in flight)
    const uint32_t sb = lds_offset(smem) + (st % kSkStages) * L::STAGE;
    uint32_t wa[2], wb[NCT][2];
    skinny_read_scales<NCT>(sb + L::A_SC + ra_ * 8, sb + L::B_SC + r * 8, wa, wb);
    u32x4 fa[4], fb[4][NCT];
    skinny_read_codes<NCT>(sb + L::A_CODES + ra_ * 128, sb + L::B_CODES + r * 128, r & 7, h, fa, fb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // lane half h holds block 2 kk + h of its row; the scale word of blocks
      // 4 (kk / 2) .. is shifted by h bytes so opsel = 2 (kk % 2) picks it
      const int sa = (int)(wa[kk >> 1] >> (8 * h));
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int sbw = (int)(wb[j][kk >> 1] >> (8 * h));
        const uint4 a4 = {fa[kk].x, fa[kk].y, fa[kk].z, fa[kk].w}, b4 = {fb[kk][j].x, fb[kk][j].y, fb[kk][j].z, fb[kk][j].w};
        acc[j] = (kk & 1) ? mfma_fp4_op<2>(a4, b4, sa, sbw, acc[j]) : mfma_fp4_op<0>(a4, b4, sa, sbw, acc[j]);
      }
    }
    // every wave is done with the buffer of stage st before it is refilled
    __asm__ volatile("" ::: "memory");
    METIS_WAIT_LDS0();
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (st + kSkStages < nst) issue(st + kSkStages);
  }
  float *o = out + (int64_t)by * rows * cols;
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int col = 32 * j + r;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t orow = row0 + 32 * wave + (q >> 2) * 8 + h * 4 + (q & 3);
      if (orow < rows && col < cols) o[orow * cols + col] = acc[j][q];
    }
  }
}

template <int NCT>
__global__ void __launch_bounds__(256)
    skinny_dma_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, int64_t rows,
                      const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs, int cols, int64_t T,
                      int64_t chunk, float *__restrict__ out) {
  skinny_dma_block<NCT>(ac, as, rows, bc, bs, cols, T, chunk, out, blockIdx.x, blockIdx.y);
}

// Up to three skinny products of one GEMM preparation (P, Q and Fa^T Fb) in
// one launch: the grid is the concatenation of their (row block, split)
// grids, so the small products run beside the large ones instead of after
// them.
struct SkinnyJob {
  const uint8_t *ac, *as, *bc, *bs;
  float *out;
  int64_t rows, chunk;
  int cols, gx, blocks;
};
struct SkinnyJobs {
  SkinnyJob job[3];
  int64_t T;
  int count;
};

template <int NCT>
__global__ void __launch_bounds__(256) skinny_dma_jobs_kernel(const SkinnyJobs jobs) {
  int b = blockIdx.x, j = 0;
  while (j + 1 < jobs.count && b >= jobs.job[j].blocks) {
    b -= jobs.job[j].blocks;
    ++j;
  }
  const SkinnyJob &q = jobs.job[j];
  skinny_dma_block<NCT>(q.ac, q.as, q.rows, q.bc, q.bs, q.cols, jobs.T, q.chunk, q.out, b % q.gx, b / q.gx);
}

// NVFP4: codes and E4M3 block scales are decoded exactly to fp16 while being
// staged into LDS (64 contraction elements per stage), multiplied on the
// fp16 32x32x16 MFMA with fp32 accumulation; the product of the two tensor
// scales multiplies the accumulators once before the correction. Thread t
// stages half (t & 1) of row t >> 1 of each operand: 32 codes, two blocks.

__global__ void __launch_bounds__(kGemmThreads, 1)
    gemm_nv_kernel(const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as, const float *__restrict__ ats,
                   int64_t M, const uint8_t *__restrict__ bc, const uint8_t *__restrict__ bs,
                   const float *__restrict__ bts, int64_t N, int64_t T, const unsigned short *__restrict__ l1,
                   const unsigned short *__restrict__ l2, int rp, float *__restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[NV_LDS];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  tile_coords(tm, tn, (int)cdiv(M, BM), (int)cdiv(N, BN));
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t nb = T / 16;
  const int nst = (int)cdiv(T, 64);
  floatx16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  uint4 ga, gb;
  uint32_t gsa, gsb;
  const int half = t & 1, rr = t >> 1;
  const int64_t ar = m0 + rr, br = n0 + rr;
  auto load_stage = [&](int st) {
    const int64_t e = (int64_t)st * 64 + half * 32;
    const bool ea = ar < M && e < T, eb = br < N && e < T;
    ga = ea ? *(const uint4 *)(ac + ar * (T / 2) + e / 2) : uint4{0u, 0u, 0u, 0u};
    gb = eb ? *(const uint4 *)(bc + br * (T / 2) + e / 2) : uint4{0u, 0u, 0u, 0u};
    gsa = ea ? ((uint32_t)as[ar * nb + e / 16] | ((uint32_t)as[ar * nb + e / 16 + 1] << 8)) : 0u;
    gsb = eb ? ((uint32_t)bs[br * nb + e / 16] | ((uint32_t)bs[br * nb + e / 16 + 1] << 8)) : 0u;
  };
  auto store_stage = [&](int buf) {
    uint8_t *A_ = smem + buf * NV_STAGE_BYTES, *B_ = A_ + BM * NV_ROWB;
    const uint32_t wa[4] = {ga.x, ga.y, ga.z, ga.w};
    const uint32_t wb[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // word w holds elements 8w .. 8w+7 of this half (block w / 2); byte p
      // of it elements 2p (low nibble) and 2p + 1. The FP4 conversion at
      // scale 1 gives the E2M1 values in fp16; the product with the E4M3
      // block scale has at most five significant bits and lies in
      // [2^-10, 2688], so the fp16 multiply is exact.
      const _Float16 fa = (_Float16)e4m3_value((gsa >> (8 * (w >> 1))) & 0xFFu);
      const _Float16 fb = (_Float16)e4m3_value((gsb >> (8 * (w >> 1))) & 0xFFu);
      const halfx2 sa2 = {fa, fa}, sb2 = {fb, fb};
      *(halfx8 *)(A_ + rr * NV_ROWB + (half * 32 + w * 8) * 2) = fp4x8_to_f16(wa[w], sa2);
      *(halfx8 *)(B_ + rr * NV_ROWB + (half * 32 + w * 8) * 2) = fp4x8_to_f16(wb[w], sb2);
    }
  };
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    if (st + 1 < nst) load_stage(st + 1);
    const uint8_t *A_ = smem + cur * NV_STAGE_BYTES, *B_ = A_ + BM * NV_ROWB;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      halfx8 a8[WM], b8[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        a8[i] = *(const halfx8 *)(A_ + (wm * 128 + i * 32 + r32) * NV_ROWB + ks * 32 + h * 16);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        b8[j] = *(const halfx8 *)(B_ + (wn * 64 + j * 32 + r32) * NV_ROWB + ks * 32 + h * 16);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8[i], b8[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < nst) store_stage(cur ^ 1);
    __syncthreads();
  }
  epilogue(acc, ats[0] * bts[0], smem, m0, n0, M, N, l1, l2, rp, C, ldc);
}

// ====================================================================== host
// The asynchronous-load skinny kernel applies: K and the split a multiple of
// 256, 16-byte aligned codes, 4-byte aligned scales, byte offsets below 2^31.
bool skinny_dma_ok(const metis_fp4_t *A, int64_t rows, const metis_fp4_t *B, int cols, int64_t T, int64_t chunk) {
  return A->fmt == METIS_MXFP4 && T % 256 == 0 && chunk % 256 == 0 &&
         (((uintptr_t)A->codes | (uintptr_t)B->codes) & 15) == 0 &&
         (((uintptr_t)A->scales | (uintptr_t)B->scales) & 3) == 0 &&
         std::max<int64_t>(rows, cols) * (T / 2) < ((int64_t)1 << 31);
}

int skinny_nct(int cols) { return cols <= 32 ? 1 : (cols <= 64 ? 2 : 3); }

void launch_skinny(const metis_fp4_t *A, int64_t rows, const metis_fp4_t *B, int cols, int64_t T, int ks,
                   int64_t chunk, float *out, hipStream_t st) {
  const dim3 grid((unsigned)cdiv(rows, 32), ks);
  const int nct = cols <= 32 ? 1 : (cols <= 64 ? 2 : 3);
  if (A->fmt == METIS_NVFP4) {
#define NV_SKINNY(N)                                                                                              \
  skinny_nv_kernel<N><<<grid, 64, 0, st>>>(A->codes, A->scales, A->tensor_scale, rows, B->codes, B->scales, \
                                           B->tensor_scale, cols, T, chunk, out)
    if (nct == 1) NV_SKINNY(1);
    else if (nct == 2) NV_SKINNY(2);
    else NV_SKINNY(3);
#undef NV_SKINNY
    return;
  }
  if (skinny_dma_ok(A, rows, B, cols, T, chunk)) {
    const dim3 g((unsigned)cdiv(rows, kSkRows), ks);
    if (nct == 1)
      skinny_dma_kernel<1><<<g, 256, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
    else if (nct == 2)
      skinny_dma_kernel<2><<<g, 256, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
    else
      skinny_dma_kernel<3><<<g, 256, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
    return;
  }
  if (nct == 1)
    skinny_kernel<1><<<grid, 64, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
  else if (nct == 2)
    skinny_kernel<2><<<grid, 64, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
  else
    skinny_kernel<3><<<grid, 64, 0, st>>>(A->codes, A->scales, rows, B->codes, B->scales, cols, T, chunk, out);
}

bool nv_scales_ok(const Side &x) {
  if (x.R->fmt != METIS_NVFP4) return true;
  if (x.rows > 0 && x.T > 0 && !x.R->tensor_scale) return false;
  return x.k == 0 || (x.F->tensor_scale && x.G->tensor_scale && x.F->fmt == METIS_NVFP4 && x.G->fmt == METIS_NVFP4);
}

metis_status_t check_pair(const Side &a, const Side &b) {
  if (a.T != b.T) return METIS_ERR_INVALID;
  if (a.R->fmt != b.R->fmt || (a.R->fmt != METIS_MXFP4 && a.R->fmt != METIS_NVFP4)) return METIS_ERR_INVALID;
  if (a.k && (a.F->fmt != a.R->fmt || a.G->fmt != a.R->fmt)) return METIS_ERR_INVALID;
  if (b.k && (b.F->fmt != b.R->fmt || b.G->fmt != b.R->fmt)) return METIS_ERR_INVALID;
  if (!nv_scales_ok(a) || !nv_scales_ok(b)) return METIS_ERR_INVALID;
  if (a.k > 96 || b.k > 96) return METIS_ERR_UNSUPPORTED;
  if (a.rows == 0 || b.rows == 0 || a.T == 0) return METIS_OK;
  if (a.R->rows != a.rows || a.R->cols != a.T || b.R->rows != b.rows || b.R->cols != b.T) return METIS_ERR_INVALID;
  const int64_t B = a.R->fmt == METIS_NVFP4 ? 16 : 32;
  if (a.T % B || (((uintptr_t)a.R->codes) & 15) || (((uintptr_t)b.R->codes) & 15)) return METIS_ERR_INVALID;
  // the NVFP4 main loop stages 32-element halves (two blocks) per row
  if (a.R->fmt == METIS_NVFP4 && a.T % 32) return METIS_ERR_UNSUPPORTED;
  return METIS_OK;
}

// Stage 1 + panels: everything the main kernel needs besides the residuals.
metis_status_t gemm_prepare(const Side &a, const Side &b, void *ws, size_t ws_bytes, hipStream_t st) {
  metis_status_t s = check_pair(a, b);
  if (s != METIS_OK) return s;
  if (a.rows == 0 || b.rows == 0 || a.T == 0 || (a.k == 0 && b.k == 0)) return METIS_OK;
  GemmPlan p = make_gemm_plan(a.rows, b.rows, a.T, a.k, b.k, ws);
  if (!ws || ws_bytes < p.bytes) return METIS_ERR_WORKSPACE;
  if (((uintptr_t)ws) & 255) return METIS_ERR_INVALID;
  {
    // the products this GEMM needs: P = Ra Fb, Q = Rb Fa, Fa^T Fb
    struct Prod {
      const metis_fp4_t *A, *B;
      int64_t rows;
      int cols, ks;
      int64_t chunk;
      float *out;
    } prods[3];
    int np = 0;
    if (b.k) prods[np++] = {a.R, b.F, a.rows, b.k, p.ks_p, p.tc_p, p.ppart};
    if (a.k) prods[np++] = {b.R, a.F, b.rows, a.k, p.ks_q, p.tc_q, p.qpart};
    if (a.k && b.k) prods[np++] = {a.F, b.F, a.k, b.k, p.ks_c, p.tc_c, p.cpart};
    bool one = np > 1;
    for (int i = 0; i < np; ++i)
      one = one && skinny_dma_ok(prods[i].A, prods[i].rows, prods[i].B, prods[i].cols, a.T, prods[i].chunk) &&
            skinny_nct(prods[i].cols) == skinny_nct(prods[0].cols);
    if (one) {
      SkinnyJobs jobs{};
      jobs.T = a.T;
      jobs.count = np;
      int64_t total = 0;
      for (int i = 0; i < np; ++i) {
        const Prod &q = prods[i];
        const int gx = (int)cdiv(q.rows, kSkRows);
        jobs.job[i] = {q.A->codes, q.A->scales, q.B->codes, q.B->scales, q.out, q.rows, q.chunk, q.cols, gx, gx * q.ks};
        total += (int64_t)gx * q.ks;
      }
      const int nct = skinny_nct(prods[0].cols);
      if (nct == 1) skinny_dma_jobs_kernel<1><<<(unsigned)total, 256, 0, st>>>(jobs);
      else if (nct == 2) skinny_dma_jobs_kernel<2><<<(unsigned)total, 256, 0, st>>>(jobs);
      else skinny_dma_jobs_kernel<3><<<(unsigned)total, 256, 0, st>>>(jobs);
    } else {
      for (int i = 0; i < np; ++i)
        launch_skinny(prods[i].A, prods[i].rows, prods[i].B, prods[i].cols, a.T, prods[i].ks, prods[i].chunk,
                      prods[i].out, st);
    }
  }
  if (a.k && b.k)
    cross_reduce_kernel<<<(unsigned)cdiv(a.k * b.k, 256), 256, 0, st>>>(p.cpart, p.ks_c, a.k * b.k, p.cross);
  const unsigned pgrid = (unsigned)(cdiv(a.rows, kPanelRows) + cdiv(b.rows, kPanelRows));
#define PANEL(NV, KM)                                                                                             \
  panel_kernel<NV, KM><<<pgrid, 256, 0, st>>>(a.rows, b.rows, a.k, b.k, p.rp, p.ppart, p.ks_p, p.qpart, p.ks_q,        \
                                         p.cross, a.S, b.S, a.k ? a.G->codes : nullptr,                            \
                                         a.k ? a.G->scales : nullptr, a.k ? a.G->tensor_scale : nullptr,           \
                                         b.k ? b.G->codes : nullptr, b.k ? b.G->scales : nullptr,                  \
                                         b.k ? b.G->tensor_scale : nullptr, p.l1, p.l2)
  const bool km64 = a.k <= 64 && b.k <= 64;
  if (a.R->fmt == METIS_NVFP4) {
    if (km64) PANEL(true, 64);
    else PANEL(true, 96);
  } else {
    if (km64) PANEL(false, 64);
    else PANEL(false, 96);
  }
#undef PANEL
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

// Main FP4 GEMM of the residuals plus the low-rank correction from the panels
// that gemm_prepare left in the same workspace.
metis_status_t gemm_main(const Side &a, const Side &b, float *C, int64_t ldc, const void *ws, size_t ws_bytes,
                         hipStream_t st) {
  metis_status_t s = check_pair(a, b);
  if (s != METIS_OK) return s;
  if (ldc < b.rows) return METIS_ERR_INVALID;
  if (a.rows == 0 || b.rows == 0) return METIS_OK;
  if (!C) return METIS_ERR_INVALID;
  int rp = 0;
  const unsigned short *l1 = nullptr, *l2 = nullptr;
  if (a.k || b.k) {
    GemmPlan p = make_gemm_plan(a.rows, b.rows, a.T, a.k, b.k, (void *)ws);
    if (!ws || ws_bytes < p.bytes) return METIS_ERR_WORKSPACE;
    if (((uintptr_t)ws) & 255) return METIS_ERR_INVALID;
    rp = p.rp;
    l1 = p.l1;
    l2 = p.l2;
  }
  const unsigned tiles = (unsigned)(cdiv(a.rows, BM) * cdiv(b.rows, BN));
  if (a.R->fmt == METIS_NVFP4 && a.T % 128 == 0 &&
      ((uintptr_t)a.R->codes | (uintptr_t)b.R->codes) % 16 == 0 &&
      std::max(a.rows, b.rows) * std::max<int64_t>(a.T / 2, 2 * (int64_t)rp) < ((int64_t)1 << 31))
    gemm_nvd_kernel<<<std::min<unsigned>(tiles, kMxMaxGrid), kMxThreads, 0, st>>>(
        a.R->codes, a.R->scales, a.R->tensor_scale, a.rows, b.R->codes, b.R->scales, b.R->tensor_scale, b.rows, a.T,
        l1, l2, rp, C, ldc);
  else if (a.R->fmt == METIS_NVFP4)
    gemm_nv_kernel<<<tiles, kGemmThreads, 0, st>>>(a.R->codes, a.R->scales, a.R->tensor_scale, a.rows, b.R->codes,
                                          b.R->scales, b.R->tensor_scale, b.rows, a.T, l1, l2, rp, C, ldc);
  else if (a.T % 512 == 0 && ((uintptr_t)a.R->codes | (uintptr_t)b.R->codes | (uintptr_t)a.R->scales |
                              (uintptr_t)b.R->scales) % 16 == 0 &&
           std::max(a.rows, b.rows) * std::max<int64_t>(a.T / 2, 2 * (int64_t)rp) < ((int64_t)1 << 31))
    gemm_mx_kernel<<<std::min<unsigned>(tiles, kMxMaxGrid), kMxThreads, 0, st>>>(
        a.R->codes, a.R->scales, a.rows, b.R->codes, b.R->scales, b.rows, a.T, l1, l2, rp, C, ldc);
  else
    gemm_mx8_kernel<<<tiles, kGemmThreads, 0, st>>>(a.R->codes, a.R->scales, a.rows, b.R->codes, b.R->scales,
                                                    b.rows, a.T, l1, l2, rp, C, ldc);
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

metis_status_t gemm_nt(const Side &a, const Side &b, float *C, int64_t ldc, void *ws, size_t ws_bytes,
                       hipStream_t st) {
  metis_status_t s = gemm_prepare(a, b, ws, ws_bytes, st);
  if (s != METIS_OK) return s;
  return gemm_main(a, b, C, ldc, ws, ws_bytes, st);
}

size_t gemm_bytes(const metis_split_t *a, bool at, const metis_split_t *b, bool bt) {
  const int64_t ra = at ? a->n : a->m, rb = bt ? b->n : b->m, T = at ? a->m : a->n;
  return make_gemm_plan(ra, rb, T, a->k, b->k, nullptr).bytes;
}

}  // namespace

extern "C" size_t metis_gemm_nt_workspace_bytes(const metis_split_t *a, int32_t a_trans, const metis_split_t *b,
                                                int32_t b_trans) {
  if (!a || !b) return 0;
  return gemm_bytes(a, a_trans != 0, b, b_trans != 0);
}

extern "C" metis_status_t metis_gemm_nt_prepare(const metis_split_t *a, int32_t a_trans, const metis_split_t *b,
                                                int32_t b_trans, void *ws, size_t ws_bytes, hipStream_t stream) {
  Side sa, sb;
  if (!a || !b || !make_side(a, a_trans != 0, sa) || !make_side(b, b_trans != 0, sb)) return METIS_ERR_INVALID;
  return gemm_prepare(sa, sb, ws, ws_bytes, stream);
}

extern "C" metis_status_t metis_gemm_nt_main(const metis_split_t *a, int32_t a_trans, const metis_split_t *b,
                                             int32_t b_trans, float *C, int64_t ldc, const void *ws, size_t ws_bytes,
                                             hipStream_t stream) {
  Side sa, sb;
  if (!a || !b || !make_side(a, a_trans != 0, sa) || !make_side(b, b_trans != 0, sb)) return METIS_ERR_INVALID;
  return gemm_main(sa, sb, C, ldc, ws, ws_bytes, stream);
}

extern "C" size_t metis_linear_workspace_bytes(const metis_split_t *X, const metis_split_t *W,
                                               const metis_split_t *dY) {
  if (!X || !W) return 0;
  size_t n = gemm_bytes(X, false, W, false);
  if (dY) {
    n = std::max(n, gemm_bytes(dY, false, W, true));
    n = std::max(n, gemm_bytes(dY, true, X, true));
  }
  return n;
}

extern "C" metis_status_t spectral_fp4_linear_fwd(const metis_split_t *X, const metis_split_t *W, float *Y,
                                                  int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!X || !W || X->n != W->n || X->k < 0 || W->k < 0) return METIS_ERR_INVALID;
  Side a, b;
  if (!make_side(X, false, a) || !make_side(W, false, b)) return METIS_ERR_INVALID;
  return gemm_nt(a, b, Y, ldy, ws, ws_bytes, stream);
}

// ------------------------------------------------- forward without allocation
// Scratch of spectral_fp4_linear_fwd_noalloc: a device array in the library's
// code object, so every GPU the library runs on holds its own copy from the
// code object's load until the process ends. Host code never passes its name
// to a kernel (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = METIS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the
// device's first call, then cached).
metis_status_t scratch_on_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return METIS_ERR_HIP;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return METIS_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return METIS_OK;
}
}  // namespace

extern "C" metis_status_t spectral_fp4_linear_fwd_noalloc(const metis_split_t *X, const metis_split_t *W, float *Y,
                                                          int64_t ldy, hipStream_t stream) {
  if (!X || !W || X->n != W->n || X->k < 0 || W->k < 0) return METIS_ERR_INVALID;
  Side a, b;
  if (!make_side(X, false, a) || !make_side(W, false, b)) return METIS_ERR_INVALID;
  const metis_status_t s = check_pair(a, b);
  if (s != METIS_OK) return s;
  const size_t need = gemm_bytes(X, false, W, false);
  if (need > kStaticScratchBytes) return METIS_ERR_TOO_LARGE;
  void *ws = nullptr;
  if (a.rows && b.rows && a.T && (a.k || b.k)) {
    const metis_status_t g = scratch_on_current_device(&ws);
    if (g != METIS_OK) return g;
  }
  return gemm_nt(a, b, Y, ldy, ws, kStaticScratchBytes, stream);
}

extern "C" metis_status_t spectral_fp4_linear_bwd(const metis_split_t *dY, const metis_split_t *X,
                                                  const metis_split_t *W, float *dX, int64_t lddx, float *dW,
                                                  int64_t lddw, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!dY || !X || !W) return METIS_ERR_INVALID;
  if (dY->m != X->m || dY->n != W->m || X->n != W->n) return METIS_ERR_INVALID;
  if (dX) {
    Side a, b;
    if (!make_side(dY, false, a) || !make_side(W, true, b)) return METIS_ERR_INVALID;
    const metis_status_t s = gemm_nt(a, b, dX, lddx, ws, ws_bytes, stream);
    if (s != METIS_OK) return s;
  }
  if (dW) {
    Side a, b;
    if (!make_side(dY, true, a) || !make_side(X, true, b)) return METIS_ERR_INVALID;
    const metis_status_t s = gemm_nt(a, b, dW, lddw, ws, ws_bytes, stream);
    if (s != METIS_OK) return s;
  }
  return METIS_OK;
}
