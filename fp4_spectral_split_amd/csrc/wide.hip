// Small-matrix stages of the randomized split for wide sketches (96 < l <= 512,
// the sparse column sampling of the "Metis" abstract with 512 sampled
// columns): the l x l matrices no longer fit one workgroup's LDS, so each
// stage is spread over many workgroups and advanced by successive launches.
//
//   wide_chol_inv  R^-1 of the Cholesky factor of an SPD Gram matrix G = R^T R
//                  (CholeskyQR, fp64): Gauss-Jordan elimination on [G | I]
//                  giving G = L D L^T and L^-1 together, R^-1 = L^-T D^-1/2.
//                  A launch takes 16 pivots: every workgroup first eliminates
//                  the 16 pivot rows among themselves in LDS (the same
//                  arithmetic in every workgroup), then applies the 16 steps
//                  to its own rows below them.
//   wide_eigh      the k largest eigenpairs of a symmetric G (fp64):
//                  Householder reduction to tridiagonal T = Q^T G Q, one launch
//                  per reflector (each launch applies the previous reflector to
//                  the rows below it, forms the next reflector from the updated
//                  row, which every workgroup computes for itself, and starts
//                  the next matrix-vector product in the same pass over each
//                  row); eigenvalues of T by multisection on Sturm counts of
//                  its LDL^T form; eigenvectors of T from twisted
//                  factorizations; x = Q z by the reflectors in reverse order.
// The narrow (l <= 96) forms of both live in split.hip. Every reduction runs
// in a fixed order, so results are bitwise reproducible.
#include <algorithm>

#include "common.hpp"
#include "wide.hpp"

using namespace metis;

namespace {

constexpr int kWT = 256;               // threads per workgroup
constexpr int kWMax = metis_wide::kWideMax;
constexpr int kWC = kWMax / 64;        // columns per lane of a row
constexpr int kPiv = 16;               // pivots per Cholesky launch

// Sum over the workgroup (kWT threads), the same bits in every thread:
// lane 0's butterfly sum of each wave, then the waves in order.
__device__ __forceinline__ double block_sum(double v, double *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kWT / 64; ++w) s += red[w];
  return s;
}

__device__ __forceinline__ double block_max(double v, double *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < kWT / 64; ++w) s = fmax(s, red[w]);
  return s;
}

// Sum over one wave, lane 0's value in every lane.
__device__ __forceinline__ double wave_sum0(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return __shfl(v, 0, 64);
}

// ============================================================ Cholesky
// C (lp x lp) starts as the upper triangle of G (zero below the diagonal and
// beyond l); aux[0] = l * 2^-52 * max diag G, the pivot floor.
__global__ void __launch_bounds__(kWT) wchol_init_kernel(const double *__restrict__ g, int l, int lp,
                                                         double *__restrict__ C, double *__restrict__ aux) {
  __shared__ double red[kWT / 64];
  const int64_t n = (int64_t)lp * lp;
  for (int64_t e = blockIdx.x * (int64_t)kWT + threadIdx.x; e < n; e += (int64_t)gridDim.x * kWT) {
    const int p = (int)(e / lp), x = (int)(e % lp);
    C[e] = (p < l && x < l && x >= p) ? g[e] : 0.0;
  }
  if (blockIdx.x == 0) {
    double md = 0.0;
    for (int i = threadIdx.x; i < l; i += kWT) md = fmax(md, g[(int64_t)i * lp + i]);
    md = block_max(md, red);
    if (threadIdx.x == 0) aux[0] = (double)l * 2.220446049250313e-16 * md;
  }
}

// Pivots j0 .. j0 + b - 1 (b <= kPiv). Row p of C holds G'[p][x] for x >= p
// (the trailing matrix) and L^-1[p][x] for x < p (unit diagonal implicit).
// Step j: every later row p loses m = G'[j][p] / d_j times row j on x >= p
// and x < j, and its L^-1 entry at j becomes -m (an absent pivot, d_j <= the
// floor, gets m = 0). The pivot rows are final once their own step is
// reached, so they go to F (read by the finish kernel, never in place: other
// workgroups are still reading C's copy); rows below them are updated in C,
// one row per wave.
__global__ void __launch_bounds__(kWT) wchol_step_kernel(double *__restrict__ C, double *__restrict__ F, int l,
                                                         int lp, int j0, const double *__restrict__ aux) {
  __shared__ double P[kPiv][kWMax];
  __shared__ double ip[kPiv];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j1 = min(j0 + kPiv, l), b = j1 - j0;
  const double tol = aux[0];
  for (int e = t; e < b * lp; e += kWT) P[e / lp][e % lp] = C[(int64_t)(j0 + e / lp) * lp + e % lp];
  __syncthreads();
  // the pivot rows among themselves
  for (int i = 0; i < b; ++i) {
    const int j = j0 + i;
    const double d = P[i][j];
    const double inv = d > tol ? 1.0 / d : 0.0;
    if (t == 0) ip[i] = inv;
    for (int e = t; e < (b - i - 1) * lp; e += kWT) {
      const int i2 = i + 1 + e / lp, x = e % lp, p = j0 + i2;
      const double m = P[i][p] * inv;
      if (x >= p || x < j) P[i2][x] = fma(-m, P[i][x], P[i2][x]);
      else if (x == j) P[i2][x] -= m;
    }
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int e = t; e < b * lp; e += kWT) F[(int64_t)(j0 + e / lp) * lp + e % lp] = P[e / lp][e % lp];
  // own rows below the pivots
  const int p = j1 + blockIdx.x * (kWT / 64) + wave;
  if (p >= l) return;
  double r[kWC];
  double *row = C + (int64_t)p * lp;
#pragma unroll
  for (int u = 0; u < kWC; ++u) {
    const int x = lane + 64 * u;
    r[u] = x < lp ? row[x] : 0.0;
  }
  for (int i = 0; i < b; ++i) {
    const int j = j0 + i;
    const double m = P[i][p] * ip[i];
#pragma unroll
    for (int u = 0; u < kWC; ++u) {
      const int x = lane + 64 * u;
      if (x < lp) {
        if (x >= p || x < j) r[u] = fma(-m, P[i][x], r[u]);
        else if (x == j) r[u] -= m;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kWC; ++u) {
    const int x = lane + 64 * u;
    if (x < lp) row[x] = r[u];
  }
}

// R^-1[i][c] = L^-1[c][i] d_c^-1/2 for i <= c < l (zero column for an absent
// pivot, zero elsewhere); info = the first absent pivot (1-based) or 0.
__global__ void __launch_bounds__(kWT) wchol_finish_kernel(const double *__restrict__ F, int l, int lp,
                                                           const double *__restrict__ aux, double *__restrict__ rinv,
                                                           int *info) {
  const double tol = aux[0];
  const int64_t n = (int64_t)lp * lp;
  for (int64_t e = blockIdx.x * (int64_t)kWT + threadIdx.x; e < n; e += (int64_t)gridDim.x * kWT) {
    const int i = (int)(e / lp), c = (int)(e % lp);
    double r = 0.0;
    if (c < l && i <= c) {
      const double d = F[(int64_t)c * lp + c];
      if (d > tol) r = (i == c ? 1.0 : F[(int64_t)c * lp + i]) / sqrt(d);
    }
    rinv[e] = r;
  }
  if (info && blockIdx.x == 0 && threadIdx.x == 0) {
    int first = 0;
    for (int c = 0; c < l && !first; ++c)
      if (!(F[(int64_t)c * lp + c] > tol)) first = c + 1;
    *info = first;
  }
}

// ============================================================ tridiagonal
// W (lp x lp) starts as the full symmetric G from its upper triangle.
__global__ void __launch_bounds__(kWT) wtri_init_kernel(const double *__restrict__ g, int l, int lp,
                                                        double *__restrict__ W) {
  const int64_t n = (int64_t)lp * lp;
  for (int64_t e = blockIdx.x * (int64_t)kWT + threadIdx.x; e < n; e += (int64_t)gridDim.x * kWT) {
    const int r = (int)(e / lp), c = (int)(e % lp);
    W[e] = (r < l && c < l) ? g[(int64_t)min(r, c) * lp + max(r, c)] : 0.0;
  }
}

// Launch j (j = -1, 0, ..., l - 3), with jn = j + 1:
//  - if j >= 0: reflector j (v_j = V[j], beta_j) is applied to the rows below
//    it: w = p - (beta_j / 2) (p . v_j) v_j with p = pbuf[j & 1] = beta_j W v_j,
//    then W <- W - v_j w^T - w v_j^T on rows and columns > j;
//  - every workgroup forms the updated row jn itself; its diagonal is d[jn],
//    and if jn <= l - 3 its part right of the diagonal, x, gives reflector jn:
//    alpha = -sign(x_0) |x|, v = x - alpha e_0, beta = 2 / v.v, e[jn] = alpha;
//    otherwise the last off-diagonal is recorded;
//  - each wave takes one row r > jn: the update above, written back, and
//    p_r = beta_jn (W v_jn)_r into pbuf[jn & 1].
// Workgroup 0 records V[jn], beta[jn], d[jn] and e[jn]. Row jn itself is not
// written (nothing reads it again), so every workgroup reads the same copy.
__global__ void __launch_bounds__(kWT) wtri_step_kernel(double *__restrict__ W, int l, int lp, int j,
                                                        double *__restrict__ V, double *__restrict__ beta,
                                                        double *__restrict__ dg, double *__restrict__ eo,
                                                        double *__restrict__ pbuf) {
  __shared__ double sv[kWMax], sw[kWMax], sx[kWMax];
  __shared__ double red[kWT / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int jn = j + 1;
  const bool apply = j >= 0;
  // ---- w of reflector j
  {
    double part = 0.0;
    for (int c = t; c < kWMax; c += kWT) {
      const bool in = apply && c > j && c < l;
      const double v = in ? V[(int64_t)j * lp + c] : 0.0;
      const double p = in ? pbuf[(int64_t)(j & 1) * lp + c] : 0.0;
      sv[c] = v;
      sw[c] = p;
      part = fma(p, v, part);
    }
    const double K = apply ? 0.5 * beta[j] * block_sum(part, red) : 0.0;
    for (int c = t; c < kWMax; c += kWT) sw[c] = fma(-K, sv[c], sw[c]);
    __syncthreads();
  }
  // ---- row jn after the update, and reflector jn from it
  const double vr_n = sv[jn], wr_n = sw[jn];
  double s2 = 0.0;
  for (int c = t; c < kWMax; c += kWT) {
    double x = 0.0;
    if (c >= jn && c < l) x = fma(-vr_n, sw[c], fma(-wr_n, sv[c], W[(int64_t)jn * lp + c]));
    sx[c] = x;
    if (c > jn) s2 = fma(x, x, s2);
  }
  const double a2 = block_sum(s2, red);  // also orders the sx writes
  const bool refl = jn <= l - 3;
  double bet = 0.0;
  if (refl) {
    const double x0 = sx[jn + 1], nrm = sqrt(a2);
    const double alpha = x0 >= 0.0 ? -nrm : nrm;
    bet = a2 > 0.0 ? 1.0 / (nrm * (nrm + fabs(x0))) : 0.0;
    __syncthreads();
    if (t == 0) sx[jn + 1] = x0 - alpha;  // sx becomes v (zero at and left of jn)
    if (blockIdx.x == 0 && t == 0) {
      beta[jn] = bet;
      eo[jn] = alpha;
    }
  }
  if (blockIdx.x == 0 && t == 0) dg[jn] = sx[jn];
  if (blockIdx.x == 0 && t == 0 && jn == l - 2) eo[jn] = sx[jn + 1];
  __syncthreads();
  if (refl && blockIdx.x == 0)
    for (int c = t; c < lp; c += kWT) V[(int64_t)jn * lp + c] = c > jn ? sx[c] : 0.0;
  // ---- the rows below jn: update, write back, next product
  const int r = jn + 1 + blockIdx.x * (kWT / 64) + wave;
  if (r >= l) return;
  double *row = W + (int64_t)r * lp;
  const double vr = sv[r], wr = sw[r];
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kWC; ++u) {
    const int c = lane + 64 * u;
    if (c > jn && c < l) {
      const double a = fma(-vr, sw[c], fma(-wr, sv[c], row[c]));
      row[c] = a;
      if (refl) acc = fma(a, sx[c], acc);
      if (c == r && jn == l - 2) dg[r] = a;  // the last diagonal (r = l - 1)
    }
  }
  if (refl) {
    const double s = wave_sum0(acc);
    if (lane == 0) pbuf[(int64_t)(jn & 1) * lp + r] = bet * s;
  }
}

// ============================================================ eigenvalues
// One step of the LDL^T pivot recurrence q' = (d - x) - e^2 / q; a pivot
// smaller than pivmin is replaced by -pivmin.
__device__ __forceinline__ double ldl_next(double dmx, double e2, double q, double pivmin) {
  q = dmx - e2 / q;
  return fabs(q) < pivmin ? -pivmin : q;
}
__device__ __forceinline__ double ldl_start(double dmx, double pivmin) { return fabs(dmx) < pivmin ? -pivmin : dmx; }

// T's diagonal and squared off-diagonals into LDS (off-diagonals at or below
// 2^-52 ||T|| set to zero), with ||T||, the Gershgorin interval and pivmin.
struct TriShared {
  double d[kWMax], e[kWMax], e2[kWMax];
  double red[kWT / 64];
  double tn, glo, ghi, pivmin;
};

__device__ void load_tri(const double *__restrict__ dg, const double *__restrict__ eo, int l, TriShared &s) {
  const int t = threadIdx.x;
  double glo = 1.0e308, ghi = -1.0e308, tn = 0.0, e2m = 0.0;
  for (int i = t; i < l; i += kWT) {
    const double rad = (i > 0 ? fabs(eo[i - 1]) : 0.0) + (i < l - 1 ? fabs(eo[i]) : 0.0);
    glo = fmin(glo, dg[i] - rad);
    ghi = fmax(ghi, dg[i] + rad);
    tn = fmax(tn, fabs(dg[i]) + rad);
    if (i < l - 1) e2m = fmax(e2m, eo[i] * eo[i]);
  }
  glo = -block_max(-glo, s.red);
  ghi = block_max(ghi, s.red);
  tn = block_max(tn, s.red);
  e2m = block_max(e2m, s.red);
  const double tol_split = 2.220446049250313e-16 * tn;
  for (int i = t; i < l; i += kWT) {
    const double e = i < l - 1 ? (fabs(eo[i]) <= tol_split ? 0.0 : eo[i]) : 0.0;
    s.d[i] = dg[i];
    s.e[i] = e;
    s.e2[i] = e * e;
  }
  if (t == 0) {
    s.tn = tn;
    s.glo = glo;
    s.ghi = ghi;
    s.pivmin = 2.2250738585072014e-308 * fmax(1.0, e2m);
  }
  __syncthreads();
}

// The k largest eigenvalues of T, one wave per eigenvalue: 64 points cut
// its bracket into 65 parts per step, nine steps (65^9 > 2^54).
__global__ void __launch_bounds__(kWT) weig_values_kernel(const double *__restrict__ dg, const double *__restrict__ eo,
                                                          int l, int k, double *__restrict__ lam,
                                                          double *__restrict__ tn_out) {
  __shared__ TriShared s;
  load_tri(dg, eo, l, s);
  const int lane = threadIdx.x & 63, rk = blockIdx.x * (kWT / 64) + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tn_out = s.tn;
  if (rk >= k) return;
  const int a = l - 1 - rk;  // ascending index
  const double pivmin = s.pivmin;
  const double pad = 8.881784197001252e-16 * fmax(fabs(s.glo), fabs(s.ghi)) + pivmin;
  double lo = s.glo - pad, hi = s.ghi + pad;
  const double fj = (double)(lane + 1) * (1.0 / 65.0);
  for (int it = 0; it < 9; ++it) {
    const double w = hi - lo, xs = fma(w, fj, lo);
    double q = ldl_start(s.d[0] - xs, pivmin);
    int cnt = q < 0.0;
    for (int i = 1; i < l; ++i) {
      q = ldl_next(s.d[i] - xs, s.e2[i - 1], q, pivmin);
      cnt += q < 0.0;
    }
    const unsigned long long bal = __ballot(cnt > a);
    const int qf = bal ? __builtin_ctzll(bal) : 64;
    const double nlo = qf > 0 ? fma(w, (double)qf * (1.0 / 65.0), lo) : lo;
    const double nhi = qf < 64 ? fma(w, (double)(qf + 1) * (1.0 / 65.0), lo) : hi;
    lo = nlo;
    hi = nhi;
  }
  if (lane == 0) lam[rk] = 0.5 * (lo + hi);
}

// ============================================================ eigenvectors
// One thread per wanted rank c < k (one workgroup): the twisted
// factorization T - lambda I = N_r D_r N_r^T at the twist r of least |gamma_r|
// gives z (z_r = 1); its top-down pivots D+ are staged in the vector's own
// column of Z and the bottom-up pivots D- in Dm. Ranks whose eigenvalues are
// closer than 1e-7 ||T|| to the previous rank's form chains, orthogonalized
// in rank order (twice). Also S, sig_inv (sigma = sqrt(lambda); 0 at or
// below 2^-24 sigma_max).
__global__ void __launch_bounds__(kWT) weig_vectors_kernel(const double *__restrict__ dg, const double *__restrict__ eo,
                                                           int l, int lp, int k, const double *__restrict__ lam,
                                                           double *__restrict__ Z, double *__restrict__ Dm,
                                                           double *__restrict__ sig_inv, float *__restrict__ S) {
  __shared__ TriShared s;
  __shared__ int chain_any;
  load_tri(dg, eo, l, s);
  const int t = threadIdx.x;
  const double pivmin = s.pivmin;
  if (t < k) {
    const int c = t;
    const double lm = lam[c];
    double dp = ldl_start(s.d[0] - lm, pivmin);
    Z[c] = dp;
    for (int q = 0; q + 1 < l; ++q) {
      dp = ldl_next(s.d[q + 1] - lm, s.e2[q], dp, pivmin);
      Z[(int64_t)(q + 1) * lp + c] = dp;
    }
    double dm = ldl_start(s.d[l - 1] - lm, pivmin);
    Dm[(int64_t)(l - 1) * lp + c] = dm;
    double gmin = fabs(Z[(int64_t)(l - 1) * lp + c] + dm - (s.d[l - 1] - lm));
    int r = l - 1;
    for (int q = l - 2; q >= 0; --q) {
      dm = ldl_next(s.d[q] - lm, s.e2[q], dm, pivmin);
      Dm[(int64_t)q * lp + c] = dm;
      const double g = fabs(Z[(int64_t)q * lp + c] + dm - (s.d[q] - lm));
      if (g < gmin) {
        gmin = g;
        r = q;
      }
    }
    double z = 1.0, nrm2 = 1.0;
    for (int q = r - 1; q >= 0; --q) {
      z = -(s.e[q] / Z[(int64_t)q * lp + c]) * z;
      Z[(int64_t)q * lp + c] = z;
      nrm2 = fma(z, z, nrm2);
    }
    Z[(int64_t)r * lp + c] = 1.0;
    z = 1.0;
    for (int q = r + 1; q < l; ++q) {
      z = -(s.e[q - 1] / Dm[(int64_t)q * lp + c]) * z;
      Z[(int64_t)q * lp + c] = z;
      nrm2 = fma(z, z, nrm2);
    }
    const double inv = 1.0 / sqrt(nrm2);
    for (int q = 0; q < l; ++q) Z[(int64_t)q * lp + c] *= inv;
  }
  if (t == 0) {
    int any = 0;
    for (int c = 1; c < k; ++c) any |= lam[c - 1] - lam[c] < 1.0e-7 * s.tn;
    chain_any = any;
  }
  __threadfence_block();
  __syncthreads();
  if (chain_any) {
    __shared__ double red2[kWT / 64];
    int start = 0;
    for (int c = 1; c < k; ++c) {
      if (!(lam[c - 1] - lam[c] < 1.0e-7 * s.tn)) {
        start = c;
        continue;
      }
      for (int pass = 0; pass < 2; ++pass) {
        for (int b = start; b < c; ++b) {
          double part = 0.0;
          for (int q = t; q < l; q += kWT) part = fma(Z[(int64_t)q * lp + b], Z[(int64_t)q * lp + c], part);
          const double dot = block_sum(part, red2);
          for (int q = t; q < l; q += kWT) Z[(int64_t)q * lp + c] = fma(-dot, Z[(int64_t)q * lp + b], Z[(int64_t)q * lp + c]);
          __threadfence_block();
          __syncthreads();
        }
        double part = 0.0;
        for (int q = t; q < l; q += kWT) part = fma(Z[(int64_t)q * lp + c], Z[(int64_t)q * lp + c], part);
        const double inv = 1.0 / sqrt(block_sum(part, red2));
        for (int q = t; q < l; q += kWT) Z[(int64_t)q * lp + c] *= inv;
        __threadfence_block();
        __syncthreads();
      }
    }
  }
  for (int c = t; c < lp; c += kWT) {
    double sg = 0.0;
    if (c < k) {
      const double smax = sqrt(fmax(lam[0], 0.0));
      sg = sqrt(fmax(lam[c], 0.0));
      if (!(sg > smax * 5.9604644775390625e-08)) sg = 0.0;
    }
    sig_inv[c] = sg > 0.0 ? 1.0 / sg : 0.0;
    if (c < k) S[c] = (float)sg;
  }
}

// x = H_0 H_1 ... H_{l-3} z for each wanted rank, one wave per vector, the
// reflectors read in reverse order (the next one loaded during the current
// one's sum). Rows of Z beyond l come out zero.
__global__ void __launch_bounds__(kWT) weig_back_kernel(double *__restrict__ Z, int l, int lp, int k,
                                                        const double *__restrict__ V,
                                                        const double *__restrict__ beta) {
  const int lane = threadIdx.x & 63, c = blockIdx.x * (kWT / 64) + (threadIdx.x >> 6);
  if (c >= k) return;
  double z[kWC], v[kWC], vn[kWC];
#pragma unroll
  for (int u = 0; u < kWC; ++u) {
    const int q = lane + 64 * u;
    z[u] = q < l ? Z[(int64_t)q * lp + c] : 0.0;
  }
  int j = l - 3;
  if (j >= 0) {
#pragma unroll
    for (int u = 0; u < kWC; ++u) {
      const int q = lane + 64 * u;
      v[u] = q < lp ? V[(int64_t)j * lp + q] : 0.0;
    }
  }
  for (; j >= 0; --j) {
    const double bj = beta[j];
#pragma unroll
    for (int u = 0; u < kWC; ++u) {
      const int q = lane + 64 * u;
      vn[u] = (j > 0 && q < lp) ? V[(int64_t)(j - 1) * lp + q] : 0.0;
    }
    double part = 0.0;
#pragma unroll
    for (int u = 0; u < kWC; ++u) part = fma(v[u], z[u], part);
    const double sc = bj * wave_sum0(part);
#pragma unroll
    for (int u = 0; u < kWC; ++u) {
      z[u] = fma(-sc, v[u], z[u]);
      v[u] = vn[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kWC; ++u) {
    const int q = lane + 64 * u;
    if (q < lp) Z[(int64_t)q * lp + c] = q < l ? z[u] : 0.0;
  }
}

}  // namespace

namespace metis_wide {

size_t aux_doubles(int lp) { return (size_t)8 * lp + 64; }

metis_status_t wide_chol_inv(const double *g, int l, int lp, double *rinv, int *info, double *C, double *F,
                             double *aux, hipStream_t st) {
  if (l < 1 || l > kWideMax || lp < l || lp > kWideMax) return METIS_ERR_UNSUPPORTED;
  const unsigned fill = (unsigned)cdiv((int64_t)lp * lp, kWT);
  wchol_init_kernel<<<fill, kWT, 0, st>>>(g, l, lp, C, aux);
  for (int j0 = 0; j0 < l; j0 += kPiv) {
    const int below = l - std::min(j0 + kPiv, l);
    const unsigned grid = (unsigned)std::max<int64_t>(1, cdiv(below, kWT / 64));
    wchol_step_kernel<<<grid, kWT, 0, st>>>(C, F, l, lp, j0, aux);
  }
  wchol_finish_kernel<<<fill, kWT, 0, st>>>(F, l, lp, aux, rinv, info);
  return hipGetLastError() == hipSuccess ? METIS_OK : METIS_ERR_HIP;
}

metis_status_t wide_eigh(const double *g, int l, int lp, int k, double *evec, double *sig_inv, float *S, double *W,
                         double *V, double *Dm, double *aux, hipStream_t st) {
  if (l < 1 || l > kWideMax || lp < l || lp > kWideMax || k < 1 || k > l || k > kWT) return METIS_ERR_UNSUPPORTED;
  double *dg = aux, *eo = aux + lp, *beta = aux + 2 * lp, *pbuf = aux + 3 * lp, *lam = aux + 5 * lp,
         *tn = aux + 6 * lp;
  const unsigned fill = (unsigned)cdiv((int64_t)lp * lp, kWT);
  wtri_init_kernel<<<fill, kWT, 0, st>>>(g, l, lp, W);
  for (int j = -1; j <= l - 3 || j == -1; ++j) {
    const int below = l - (j + 2);
    const unsigned grid = (unsigned)std::max<int64_t>(1, cdiv(std::max(below, 0), kWT / 64));
    wtri_step_kernel<<<grid, kWT, 0, st>>>(W, l, lp, j, V, beta, dg, eo, pbuf);
  }
  weig_values_kernel<<<(unsigned)cdiv(k, kWT / 64), kWT, 0, st>>>(dg, eo, l, k, lam, tn);
  weig_vectors_kernel<<<1, kWT, 0, st>>>(dg, eo, l, lp, k, lam, evec, Dm, sig_inv, S);
  weig_back_kernel<<<(unsigned)cdiv(k, kWT / 64), kWT, 0, st>>>(evec, l, lp, k, V, beta);
  return hipGetLastError() == hipSuccess ? METIS_OK : METIS_ERR_HIP;
}

}  // namespace metis_wide
