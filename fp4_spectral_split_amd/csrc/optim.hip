// Optimizer-side terms of Metis (SII open-source-week post on Metis, §2
// "architecture" strategies 2 and 3 and §2.4 items 2 and 3; the earlier
// version's abstract on the chatpaper.ai page, items (ii) and (iii)). The
// pages describe both in words only; the forms implemented are these:
//
//   spectral learning rate  on the split G = U diag(S) V^T + R of a gradient,
//                           directions below a reference rank r are scaled by
//                           gamma_i = min(gamma_max, S[r] / S_i):
//                           G <- G + U diag(S (gamma - 1)) V^T, R untouched.
//   dual-range regularizer  loss = lam_hi sum relu(|w| - tau_hi)^2
//                                + lam_lo sum_{w != 0} relu(tau_lo - |w|)^2
//                           and its gradient, both streaming passes.
#include <algorithm>

#include "common.hpp"

using namespace metis;

namespace {

constexpr int kThreads = 256;
constexpr int kRegGrid = 2048;  // workgroups of the regularizer pass (one fp64 loss partial each)

// Eight elements of a row as fp32, from one 16-byte (bf16) or two 16-byte
// (fp32) loads.
__device__ __forceinline__ void load8(const unsigned short *p, float (&v)[8]) {
  const uint4 q = *(const uint4 *)p;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
  const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Loss and gradient of the regularizer over rows x cols (cols % 8 == 0),
// eight consecutive elements of a row per thread and step. The gradient of
// an element is evaluated in fp64 in the order
//   ((2 lam_hi) relu(|w| - tau_hi)) s - ((2 lam_lo) relu(tau_lo - |w|)) s
// (s = sign(w), no fused operations) and rounded once to fp32; with
// accumulate it is added to the fp32 gradient in fp64 and rounded once.
// Each workgroup leaves one fp64 loss partial (its threads in order).
template <typename T>
__global__ void __launch_bounds__(kThreads)
    dual_range_kernel(const T *__restrict__ W, int64_t rows, int64_t cols, int64_t ldw, double tau_lo, double tau_hi,
                      double lam_lo, double lam_hi, float *__restrict__ grad, int64_t ldg, int accumulate,
                      double *__restrict__ part) {
  __shared__ double red[kThreads / 64];
  const int64_t per_row = cols / 8, total = rows * per_row;
  const double two_hi = 2.0 * lam_hi, two_lo = 2.0 * lam_lo;
  double loss = 0.0;
  for (int64_t v = blockIdx.x * (int64_t)kThreads + threadIdx.x; v < total; v += (int64_t)gridDim.x * kThreads) {
    const int64_t r = v / per_row, c = (v - r * per_row) * 8;
    float w[8];
    load8(W + r * ldw + c, w);
    float g0[8];
    if (grad && accumulate) {
      const float4 a = *(const float4 *)(grad + r * ldg + c), b = *(const float4 *)(grad + r * ldg + c + 4);
      g0[0] = a.x; g0[1] = a.y; g0[2] = a.z; g0[3] = a.w;
      g0[4] = b.x; g0[5] = b.y; g0[6] = b.z; g0[7] = b.w;
    }
    float g[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double x = (double)w[i], a = fabs(x);
      const double s = x > 0.0 ? 1.0 : (x < 0.0 ? -1.0 : 0.0);
      const double hi = fmax(__dsub_rn(a, tau_hi), 0.0);
      const double lo = a > 0.0 ? fmax(__dsub_rn(tau_lo, a), 0.0) : 0.0;
      loss = __dadd_rn(loss, __dadd_rn(__dmul_rn(lam_hi, __dmul_rn(hi, hi)), __dmul_rn(lam_lo, __dmul_rn(lo, lo))));
      const double d = __dsub_rn(__dmul_rn(__dmul_rn(two_hi, hi), s), __dmul_rn(__dmul_rn(two_lo, lo), s));
      g[i] = accumulate ? (float)__dadd_rn((double)g0[i], d) : (float)d;
    }
    if (grad) {
      *(float4 *)(grad + r * ldg + c) = make_float4(g[0], g[1], g[2], g[3]);
      *(float4 *)(grad + r * ldg + c + 4) = make_float4(g[4], g[5], g[6], g[7]);
    }
  }
  if (part) {
    loss = wave_sum_f64(loss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = loss;
    __syncthreads();
    if (threadIdx.x == 0) {
      double s = 0.0;
      for (int w = 0; w < kThreads / 64; ++w) s += red[w];
      part[blockIdx.x] = s;
    }
  }
}

// loss = the partials summed in order (one workgroup; each thread a strided
// share in order, then the threads in order).
__global__ void __launch_bounds__(kThreads) sum_partials_kernel(const double *__restrict__ part, int n,
                                                                double *__restrict__ loss) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kThreads; ++i) t += red[i];
    *loss = t;
  }
}

// ------------------------------------------------------- spectral rescale
constexpr int kLrTile = 64;
constexpr int kLrMaxK = 96;

// G[i][j] += sum_t U[i][t] c_t V[j][t] with c_t = S_t (gamma_t - 1) on a
// 64 x 64 tile per workgroup (4 x 4 outputs per thread): U and c V of the
// tile's rows staged in LDS, the sum over t in fp32 FMAs in ascending t,
// then one fp32 addition to G. gamma is recomputed by every workgroup from
// S (k <= 96 values).
__global__ void __launch_bounds__(kThreads)
    spectral_lr_kernel(float *__restrict__ G, int64_t m, int64_t n, int64_t ldg, const float *__restrict__ U,
                       const float *__restrict__ S, const float *__restrict__ V, int k, int r_ref, float gamma_max) {
  __shared__ float us[kLrTile][kLrMaxK + 1], vs[kLrTile][kLrMaxK + 1];
  __shared__ float cs[kLrMaxK];
  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int64_t i0 = (int64_t)blockIdx.y * kLrTile, j0 = (int64_t)blockIdx.x * kLrTile;
  if (t < k) {
    // gamma_t = min(gamma_max, max(1, S[r] / S_t)); c_t = S_t (gamma_t - 1)
    const float s = S[t], ref = S[r_ref];
    float c = 0.0f;
    if (s > 0.0f) {
      const float gm = fminf(gamma_max, fmaxf(1.0f, __fdiv_rn(ref, s)));
      c = s * (gm - 1.0f);
    }
    cs[t] = c;
  }
  __syncthreads();
  for (int e = t; e < kLrTile * k; e += kThreads) {
    const int rr = e / k, q = e - rr * k;
    const int64_t ri = min(i0 + rr, m - 1), rj = min(j0 + rr, n - 1);
    us[rr][q] = U[ri * k + q];
    vs[rr][q] = V[rj * k + q] * cs[q];
  }
  __syncthreads();
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
  for (int q = 0; q < k; ++q) {
    float u[4], v[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u[a] = us[ti * 4 + a][q];
      v[a] = vs[tj * 4 + a][q];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(u[a], v[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t i = i0 + ti * 4 + a;
    if (i >= m) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = j0 + tj * 4 + b;
      if (j < n) G[i * ldg + j] += acc[a][b];
    }
  }
}

}  // namespace

extern "C" size_t metis_dual_range_workspace_bytes(void) { return (size_t)kRegGrid * sizeof(double); }

extern "C" metis_status_t metis_dual_range_reg(const void *W, metis_dtype_t dt, int64_t rows, int64_t cols,
                                               int64_t ldw, float tau_lo, float tau_hi, float lam_lo, float lam_hi,
                                               float *grad, int64_t ldg, int32_t accumulate, double *loss, void *ws,
                                               size_t ws_bytes, hipStream_t stream) {
  if (dt != METIS_F32 && dt != METIS_BF16) return METIS_ERR_INVALID;
  if (rows < 0 || cols < 0 || cols % 8 || ldw < cols || (grad && ldg < cols)) return METIS_ERR_INVALID;
  if (!(tau_lo >= 0.0f) || !(tau_hi >= tau_lo) || !(lam_lo >= 0.0f) || !(lam_hi >= 0.0f)) return METIS_ERR_INVALID;
  const int elem = dt == METIS_F32 ? 4 : 2;
  if (rows && cols && (!W || ((uintptr_t)W & 15) || (ldw * elem) % 16)) return METIS_ERR_INVALID;
  if (grad && rows && cols && (((uintptr_t)grad & 15) || (ldg * 4) % 16)) return METIS_ERR_INVALID;
  if (loss && (!ws || ws_bytes < metis_dual_range_workspace_bytes())) return METIS_ERR_WORKSPACE;
  if (loss && ((uintptr_t)ws & 7)) return METIS_ERR_INVALID;
  double *part = loss ? (double *)ws : nullptr;
  const int64_t vecs = rows * (cols / 8);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(kRegGrid, cdiv(vecs, kThreads)));
  if (dt == METIS_F32)
    dual_range_kernel<float><<<grid, kThreads, 0, stream>>>((const float *)W, rows, cols, ldw, tau_lo, tau_hi,
                                                             lam_lo, lam_hi, grad, ldg, accumulate, part);
  else
    dual_range_kernel<unsigned short><<<grid, kThreads, 0, stream>>>((const unsigned short *)W, rows, cols, ldw,
                                                                      tau_lo, tau_hi, lam_lo, lam_hi, grad, ldg,
                                                                      accumulate, part);
  if (loss) sum_partials_kernel<<<1, kThreads, 0, stream>>>(part, (int)grid, loss);
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

extern "C" metis_status_t metis_spectral_lr_rescale(float *G, int64_t m, int64_t n, int64_t ldg, const float *U,
                                                    const float *S, const float *V, int32_t k, int32_t r_ref,
                                                    float gamma_max, hipStream_t stream) {
  if (m < 0 || n < 0 || ldg < n) return METIS_ERR_INVALID;
  if (k < 1 || r_ref < 0 || r_ref >= k || !(gamma_max >= 1.0f)) return METIS_ERR_INVALID;
  if (k > kLrMaxK) return METIS_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return METIS_OK;
  if (!G || !U || !S || !V) return METIS_ERR_INVALID;
  const dim3 grid((unsigned)cdiv(n, kLrTile), (unsigned)cdiv(m, kLrTile));
  spectral_lr_kernel<<<grid, kThreads, 0, stream>>>(G, m, n, ldg, U, S, V, k, r_ref, gamma_max);
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}
