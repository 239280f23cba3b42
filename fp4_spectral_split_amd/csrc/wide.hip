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
constexpr int kPiv = 16;               // pivots per Cholesky launch

// Sum over the workgroup (kWT threads), the same bits in every thread: each
// wave's DPP sum (wave_sum_f64), then the waves in order.
__device__ __forceinline__ double block_sum(double v, double *red) {
  v = wave_sum_f64(v);
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

// Sum over one wave, the same bits in every lane.
__device__ __forceinline__ double wave_sum0(double v) { return wave_sum_f64(v); }

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
// NC = lp / 64 columns per lane, fixed at compile time: every load takes an
// always-valid address and every per-element condition is a select, so no
// branch separates a load from its use.
template <int NC>
__global__ void __launch_bounds__(kWT) wchol_step_kernel(double *__restrict__ C, double *__restrict__ F, int l,
                                                         int j0, const double *__restrict__ aux) {
  constexpr int lp = NC * 64;
  __shared__ double P[kPiv][lp];
  __shared__ double ip[kPiv];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int j1 = min(j0 + kPiv, l), b = j1 - j0;
  const double tol = aux[0];
  // own row below the pivots (one per wave), loaded with the pivot rows
  const int p = j1 + blockIdx.x * (kWT / 64) + wave;
  const bool own = p < l;
  double *row = C + (int64_t)(own ? p : 0) * lp;
  double r[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) r[u] = row[lane + 64 * u];
  // pivot rows (rows past the block repeat its last row: same values)
  double pr[4][NC];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const int i = min(wave + 4 * k4, b - 1);
#pragma unroll
    for (int u = 0; u < NC; ++u) pr[k4][u] = C[(int64_t)(j0 + i) * lp + lane + 64 * u];
  }
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const int i = min(wave + 4 * k4, b - 1);
#pragma unroll
    for (int u = 0; u < NC; ++u) P[i][lane + 64 * u] = pr[k4][u];
  }
  __syncthreads();
  // the pivot rows among themselves, a row per wave
  for (int i = 0; i < b; ++i) {
    const int j = j0 + i;
    const double d = P[i][j];
    const double inv = d > tol ? 1.0 / d : 0.0;
    if (t == 0) ip[i] = inv;
    for (int i2 = i + 1 + wave; i2 < b; i2 += kWT / 64) {
      const int q = j0 + i2;
      const double m = P[i][q] * inv;
      double pi[NC], p2[NC];
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        pi[u] = P[i][lane + 64 * u];
        p2[u] = P[i2][lane + 64 * u];
      }
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int x = lane + 64 * u;
        const double mm = (x >= q || x < j) ? m : 0.0;
        P[i2][x] = fma(-mm, pi[u], p2[u]) - (x == j ? m : 0.0);
      }
    }
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int i = wave; i < b; i += kWT / 64)
#pragma unroll
      for (int u = 0; u < NC; ++u) F[(int64_t)(j0 + i) * lp + lane + 64 * u] = P[i][lane + 64 * u];
  if (!own) return;
  for (int i = 0; i < b; ++i) {
    const int j = j0 + i;
    const double m = P[i][p] * ip[i];
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int x = lane + 64 * u;
      const double mm = (x >= p || x < j) ? m : 0.0;
      r[u] = fma(-mm, P[i][x], r[u]) - (x == j ? m : 0.0);
    }
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) row[lane + 64 * u] = r[u];
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
  if (info && blockIdx.x == 0) {
    // first absent pivot: the least absent index over the workgroup
    __shared__ int firsts[kWT / 64];
    int first = 0x7FFFFFFF;
    for (int c = threadIdx.x; c < l; c += kWT)
      if (!(F[(int64_t)c * lp + c] > tol)) first = min(first, c);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
    if ((threadIdx.x & 63) == 0) firsts[threadIdx.x >> 6] = first;
    __syncthreads();
    if (threadIdx.x == 0) {
      int f = firsts[0];
      for (int w = 1; w < kWT / 64; ++w) f = min(f, firsts[w]);
      *info = f == 0x7FFFFFFF ? 0 : f + 1;
    }
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
template <int NC>
__global__ void __launch_bounds__(kWT) wtri_step_kernel(double *__restrict__ W, int l, int j, double *__restrict__ V,
                                                        double *__restrict__ beta, double *__restrict__ dg,
                                                        double *__restrict__ eo, double *__restrict__ pbuf) {
  constexpr int lp = NC * 64;
  __shared__ double sv[lp], sw[lp], sx[lp];
  __shared__ double red[kWT / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int jn = j + 1;
  const bool apply = j >= 0;
  // every global load of the launch is issued here, before any is used:
  // reflector j and p_j, row jn (clamped addresses, masked values), the
  // wave's own row
  constexpr int PC = (lp + kWT - 1) / kWT;
  const int js = max(j, 0);
  double lv[PC], lq[PC], lx[PC];
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int c = min(t + kWT * u, lp - 1);
    lv[u] = V[(int64_t)js * lp + c];
    lq[u] = pbuf[(int64_t)(js & 1) * lp + c];
    lx[u] = W[(int64_t)jn * lp + c];
  }
  const double bj = beta[js];
  const int r = jn + 1 + blockIdx.x * (kWT / 64) + wave;
  const bool own = r < l;
  double *row = W + (int64_t)(own ? r : jn) * lp;
  double a[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) a[u] = row[lane + 64 * u];
  // ---- w of reflector j: w = p - (beta_j / 2) (p . v) v
  double part = 0.0;
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int c = t + kWT * u;
    const bool in = apply && c > j && c < l;
    lv[u] = in ? lv[u] : 0.0;
    lq[u] = in ? lq[u] : 0.0;
    if (c < lp) sv[c] = lv[u];
    part = fma(lq[u], lv[u], part);
  }
  const double K = apply ? 0.5 * bj * block_sum(part, red) : 0.0;
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int c = t + kWT * u;
    if (c < lp) sw[c] = fma(-K, lv[u], lq[u]);
  }
  __syncthreads();
  // ---- row jn after the update, and reflector jn from it
  const double vr_n = sv[jn], wr_n = sw[jn];
  double s2 = 0.0;
#pragma unroll
  for (int u = 0; u < PC; ++u) {
    const int c = t + kWT * u;
    if (c < lp) {
      const double x = (c >= jn && c < l) ? fma(-vr_n, sw[c], fma(-wr_n, sv[c], lx[u])) : 0.0;
      sx[c] = x;
      s2 = fma(c > jn ? x : 0.0, x, s2);
    }
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
  if (!own) return;
  const double vr = sv[r], wr = sw[r];
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int c = lane + 64 * u;
    const bool in = c > jn && c < l;
    const double x = in ? fma(-vr, sw[c], fma(-wr, sv[c], a[u])) : a[u];
    a[u] = x;
    acc = fma(in ? x : 0.0, sx[c], acc);
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) row[lane + 64 * u] = a[u];
  if (jn == l - 2) {
    // the last diagonal (r = l - 1)
#pragma unroll
    for (int u = 0; u < NC; ++u)
      if (lane + 64 * u == r) dg[r] = a[u];
  }
  if (refl) {
    const double s = wave_sum0(acc);
    if (lane == 0) pbuf[(int64_t)(jn & 1) * lp + r] = bet * s;
  }
}

// ============================================================ eigenvalues
// 1 / q from the hardware estimate (about 2^-25 relative) and two Newton
// steps: correct to about 2^-52.
__device__ __forceinline__ double recip(double q) {
  double r = __builtin_amdgcn_rcp(q);
  r = fma(r, fma(-q, r, 1.0), r);
  return fma(r, fma(-q, r, 1.0), r);
}

// One step of the LDL^T pivot recurrence q' = (d - x) - e^2 / q; a pivot
// smaller than pivmin is replaced by -pivmin. The counts take one Newton
// step on the reciprocal estimate (about 2^-50).
__device__ __forceinline__ double ldl_next(double dmx, double e2, double q, double pivmin) {
  double rq = __builtin_amdgcn_rcp(q);
  rq = fma(rq, fma(-q, rq, 1.0), rq);
  q = fma(-e2, rq, dmx);
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
// its bracket into 65 parts per step, nine steps (65^9 > 2^54). The count at
// a point x is the number of eigenvalues below x: the sign changes along the
// leading minors p_i = det(T_i - x I) of each block of T (Sturm), with
// p_i = (d_i - x) p_{i-1} - e_{i-1}^2 p_{i-2} from p = 1 at the block's start,
// summed over the blocks (T splits where an off-diagonal was set to zero).
// T is scaled by a power of two at or above ||T|| (exact), and the last two
// minors are rescaled by a power of two every eight steps. A minor that is
// exactly zero counts as positive: inside a block the next minor,
// -e^2 p_{i-2}, gives the same total as any other sign convention, and at a
// block's end it leaves an eigenvalue equal to x uncounted. The dependence
// chain holds one fused multiply-add per step.
__global__ void __launch_bounds__(kWT) weig_values_kernel(const double *__restrict__ dg, const double *__restrict__ eo,
                                                          int l, int k, double *__restrict__ lam,
                                                          double *__restrict__ tn_out) {
  __shared__ TriShared s;
  __shared__ double2 sde[kWMax];  // (d_i, e_{i-1}^2) scaled
  __shared__ int bstart[kWMax + 1], nblk;
  load_tri(dg, eo, l, s);
  const int ex = s.tn > 0.0 ? __builtin_amdgcn_frexp_exp(s.tn) : 0;  // ||T|| < 2^ex
  for (int i = threadIdx.x; i < l; i += kWT)
    sde[i] = make_double2(ldexp(s.d[i], -ex), i > 0 ? ldexp(s.e2[i - 1], -2 * ex) : 0.0);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    // block starts in order: position 0 and every i with e_{i-1} = 0
    int base = 0;
    for (int i0 = 0; i0 < l; i0 += 64) {
      const int i = i0 + lane;
      const bool st = i < l && (i == 0 || s.e2[i - 1] == 0.0);
      const unsigned long long m = __ballot(st);
      if (st) bstart[base + __popcll(m & ((1ull << lane) - 1ull))] = i;
      base += __popcll(m);
    }
    if (lane == 0) {
      nblk = base;
      bstart[base] = l;
    }
  }
  __syncthreads();
  const int rk = blockIdx.x * (kWT / 64) + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) *tn_out = s.tn;
  if (rk >= k) return;
  const int a = l - 1 - rk;  // ascending index
  const int nb = nblk;
  const double pivmin = s.pivmin;
  const double pad = 8.881784197001252e-16 * fmax(fabs(s.glo), fabs(s.ghi)) + pivmin;
  double lo = s.glo - pad, hi = s.ghi + pad;
  const double fj = (double)(lane + 1) * (1.0 / 65.0);
  for (int it = 0; it < 9; ++it) {
    const double w = hi - lo, xs = ldexp(fma(w, fj, lo), -ex);
    int cnt = 0;
    for (int b = 0; b < nb; ++b) {
      const int i1 = bstart[b + 1];
      int i = bstart[b];
      double pm = 0.0, pc = 1.0;
      auto step = [&](double2 de) {
        const double pn = fma(de.x - xs, pc, -(de.y * pm));
        cnt += (pn < 0.0) != (pc < 0.0);
        pm = pc;
        pc = pn;
      };
      for (; i + 8 <= i1; i += 8) {
        double2 de[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) de[u] = sde[i + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) step(de[u]);
        const int e = max(__builtin_amdgcn_frexp_exp(pc), __builtin_amdgcn_frexp_exp(pm));
        pc = ldexp(pc, -e);
        pm = ldexp(pm, -e);
      }
      for (; i < i1; ++i) step(sde[i]);
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
    double *zc = Z + c, *mc = Dm + c;
    double dp = ldl_start(s.d[0] - lm, pivmin);
    zc[0] = dp;
    for (int q = 0; q + 1 < l; ++q) {
      dp = ldl_next(s.d[q + 1] - lm, s.e2[q], dp, pivmin);
      zc[(int64_t)(q + 1) * lp] = dp;
    }
    // bottom-up pivots and the twist; D+ read back eight rows at a time
    double dm = ldl_start(s.d[l - 1] - lm, pivmin);
    mc[(int64_t)(l - 1) * lp] = dm;
    double gmin = fabs(dp + dm - (s.d[l - 1] - lm));
    int r = l - 1;
    for (int q0 = l - 2; q0 >= 0; q0 -= 8) {
      double pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = q0 - u >= 0 ? zc[(int64_t)(q0 - u) * lp] : 1.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 - u;
        if (q >= 0) {
          dm = ldl_next(s.d[q] - lm, s.e2[q], dm, pivmin);
          mc[(int64_t)q * lp] = dm;
          const double g = fabs(pv[u] + dm - (s.d[q] - lm));
          if (g < gmin) {
            gmin = g;
            r = q;
          }
        }
      }
    }
    double z = 1.0, nrm2 = 1.0;
    for (int q0 = r - 1; q0 >= 0; q0 -= 8) {
      double pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = q0 - u >= 0 ? zc[(int64_t)(q0 - u) * lp] : 1.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 - u;
        if (q >= 0) {
          z = -(s.e[q] * recip(pv[u])) * z;
          zc[(int64_t)q * lp] = z;
          nrm2 = fma(z, z, nrm2);
        }
      }
    }
    zc[(int64_t)r * lp] = 1.0;
    z = 1.0;
    for (int q0 = r + 1; q0 < l; q0 += 8) {
      double mv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mv[u] = q0 + u < l ? mc[(int64_t)(q0 + u) * lp] : 1.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u;
        if (q < l) {
          z = -(s.e[q - 1] * recip(mv[u])) * z;
          zc[(int64_t)q * lp] = z;
          nrm2 = fma(z, z, nrm2);
        }
      }
    }
    const double inv = 1.0 / sqrt(nrm2);
    for (int q = 0; q < l; ++q) zc[(int64_t)q * lp] *= inv;
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

// The same eigenvectors for l <= kNarrow, with the pivots in registers: for
// rank c, thread c (waves 0 and 1) runs the top-down pivots D+ and thread
// 128 + c (waves 2 and 3) the bottom-up pivots D-, both at once. D+ goes
// through LDS to the bottom-up thread, which finds the twist r (least
// |D+_q + D-_q - (d_q - lambda)|, lowest q on ties); then the top-down
// thread forms z above r (z_q = -(e_q / D+_q) z_{q+1}) and the bottom-up
// thread z from r down (z_r = 1, z_q = -(e_{q-1} / D-_q) z_{q-1}), in LDS.
// Normalization, chains and the outputs as in weig_vectors_kernel.
constexpr int kNarrow = 96;
__global__ void __launch_bounds__(kWT) neig_vectors_kernel(const double *__restrict__ dg, const double *__restrict__ eo,
                                                           int l, int lp, int k, const double *__restrict__ lam,
                                                           double *__restrict__ Z, double *__restrict__ sig_inv,
                                                           float *__restrict__ S) {
  __shared__ TriShared s;
  __shared__ double Zs[kNarrow][kNarrow + 1];
  __shared__ double nz_part[2][kNarrow];
  __shared__ int twist[kNarrow];
  __shared__ int chain_any;
  static_assert(kWT == 256 && kNarrow <= 128, "two roles of 128 threads");
  load_tri(dg, eo, l, s);
  const int t = threadIdx.x;
  const bool down = t >= 128;
  const int c = down ? t - 128 : t;
  const bool act = c < k;
  const double pivmin = s.pivmin;
  const double lm = act ? lam[c] : 0.0;
  double P[kNarrow];  // D+ (top-down thread) or D- (bottom-up thread), then z
  if (!down) {
    double dp = 0.0;
#pragma unroll
    for (int q = 0; q < kNarrow; ++q)
      if (q < l) {
        const double dmx = s.d[q] - lm;
        dp = q == 0 ? ldl_start(dmx, pivmin) : ldl_next(dmx, s.e2[q - 1], dp, pivmin);
        P[q] = dp;
        if (act) Zs[q][c] = dp;
      }
  } else {
    double dm = 0.0;
#pragma unroll
    for (int q = kNarrow - 1; q >= 0; --q)
      if (q < l) {
        const double dmx = s.d[q] - lm;
        dm = q == l - 1 ? ldl_start(dmx, pivmin) : ldl_next(dmx, s.e2[q], dm, pivmin);
        P[q] = dm;
      }
  }
  __syncthreads();
  if (down && act) {
    double gbest = 1.0e308;
    int r = 0;
#pragma unroll
    for (int q = kNarrow - 1; q >= 0; --q)
      if (q < l) {
        const double g = fabs(Zs[q][c] + P[q] - (s.d[q] - lm));
        if (g <= gbest) {
          gbest = g;
          r = q;
        }
      }
    twist[c] = r;
  }
  __syncthreads();
  if (act) {
    const int r = twist[c];
    double z = 1.0, nz = 0.0;
    if (!down) {
      // rows above the twist, from r - 1 up to 0
#pragma unroll
      for (int q = kNarrow - 2; q >= 0; --q)
        if (q + 1 < l) {
          const double f = -(s.e[q] * recip(P[q]));
          if (q < r) {
            z = f * z;
            Zs[q][c] = z;
            nz = fma(z, z, nz);
          }
        }
    } else {
      Zs[r][c] = 1.0;
      nz = 1.0;
#pragma unroll
      for (int q = 1; q < kNarrow; ++q)
        if (q < l) {
          const double f = -(s.e[q - 1] * recip(P[q]));
          if (q > r) {
            z = f * z;
            Zs[q][c] = z;
            nz = fma(z, z, nz);
          }
        }
    }
    nz_part[down][c] = nz;
  }
  __syncthreads();
  for (int e = t; e < l * k; e += kWT) {
    const int q = e / k, cc = e - (e / k) * k;
    Zs[q][cc] *= 1.0 / sqrt(nz_part[1][cc] + nz_part[0][cc]);
  }
  if (t == 0) {
    int any = 0;
    for (int cc = 1; cc < k; ++cc) any |= lam[cc - 1] - lam[cc] < 1.0e-7 * s.tn;
    chain_any = any;
  }
  __syncthreads();
  if (chain_any) {
    __shared__ double red2[kWT / 64];
    int start = 0;
    for (int cc = 1; cc < k; ++cc) {
      if (!(lam[cc - 1] - lam[cc] < 1.0e-7 * s.tn)) {
        start = cc;
        continue;
      }
      for (int pass = 0; pass < 2; ++pass) {
        for (int b = start; b < cc; ++b) {
          const double dot = block_sum(t < l ? Zs[t][b] * Zs[t][cc] : 0.0, red2);
          if (t < l) Zs[t][cc] = fma(-dot, Zs[t][b], Zs[t][cc]);
          __syncthreads();
        }
        const double inv = 1.0 / sqrt(block_sum(t < l ? Zs[t][cc] * Zs[t][cc] : 0.0, red2));
        if (t < l) Zs[t][cc] *= inv;
        __syncthreads();
      }
    }
  }
  for (int e = t; e < lp * k; e += kWT) {
    const int q = e / k, cc = e - (e / k) * k;
    Z[(int64_t)q * lp + cc] = q < l ? Zs[q][cc] : 0.0;
  }
  for (int cc = t; cc < lp; cc += kWT) {
    double sg = 0.0;
    if (cc < k) {
      const double smax = sqrt(fmax(lam[0], 0.0));
      sg = sqrt(fmax(lam[cc], 0.0));
      if (!(sg > smax * 5.9604644775390625e-08)) sg = 0.0;
    }
    sig_inv[cc] = sg > 0.0 ? 1.0 / sg : 0.0;
    if (cc < k) S[cc] = (float)sg;
  }
}

// x = H_0 H_1 ... H_{l-3} z for each wanted rank, one wave per vector
// (NC = lp / 64 rounded up rows per lane), the reflectors read in reverse
// order, D of them loaded ahead of the one being applied. Rows of Z beyond l
// come out zero.
template <int NC>
__global__ void __launch_bounds__(kWT) weig_back_kernel(double *__restrict__ Z, int l, int lp, int k,
                                                        const double *__restrict__ V,
                                                        const double *__restrict__ beta) {
  const int lane = threadIdx.x & 63, c = blockIdx.x * (kWT / 64) + (threadIdx.x >> 6);
  if (c >= k) return;
  constexpr int D = NC <= 2 ? 16 : 4;
  double z[NC], v[D][NC], bt[D];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int q = lane + 64 * u;
    z[u] = q < l ? Z[(int64_t)q * lp + c] : 0.0;
  }
  auto load = [&](int j, double (&dst)[NC], double &b) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int q = lane + 64 * u;
      dst[u] = (j >= 0 && q < lp) ? V[(int64_t)j * lp + q] : 0.0;
    }
    b = j >= 0 ? beta[j] : 0.0;
  };
  const int j_top = l - 3;
#pragma unroll
  for (int d = 0; d < D; ++d) load(j_top - d, v[d], bt[d]);
  for (int j0 = j_top; j0 >= 0; j0 -= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 - d;
      if (j >= 0) {
        double part = 0.0;
#pragma unroll
        for (int u = 0; u < NC; ++u) part = fma(v[d][u], z[u], part);
        const double sc = bt[d] * wave_sum0(part);
#pragma unroll
        for (int u = 0; u < NC; ++u) z[u] = fma(-sc, v[d][u], z[u]);
      }
      load(j - D, v[d], bt[d]);
    }
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int q = lane + 64 * u;
    if (q < lp) Z[(int64_t)q * lp + c] = q < l ? z[u] : 0.0;
  }
}

template <int NC>
void launch_back(double *Z, int l, int lp, int k, const double *V, const double *beta, hipStream_t st) {
  weig_back_kernel<NC><<<(unsigned)cdiv(k, kWT / 64), kWT, 0, st>>>(Z, l, lp, k, V, beta);
}

// out[r][c] = (sum_q x[r][q] E[q][c]) * colscale[c] for r < rows, c < k,
// fp64 sums over q in order, rounded once to fp32: 64 x 64 tiles of out, x
// and E staged through LDS 32 q at a time, 4 x 4 outputs per thread. With
// am_val, the tile's argmax of |out[:, c]| (lowest row on ties) goes to
// am_val / am_idx[tile row * k + c].
__global__ void __launch_bounds__(kWT) wassemble_kernel(const float *__restrict__ x, int64_t rows, int l, int lp,
                                                        int k, const double *__restrict__ E,
                                                        const double *__restrict__ colscale, float *__restrict__ out,
                                                        float *__restrict__ am_val, int *__restrict__ am_idx) {
  __shared__ double xs[64][33];
  __shared__ double es[32][65];
  __shared__ float bvs[16][64], bsg[16][64];
  __shared__ int bis[16][64];
  const int t = threadIdx.x, ti = t >> 4, tj = t & 15;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int q0 = 0; q0 < l; q0 += 32) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = t + kWT * u, rr = e >> 5, qq = e & 31;
      const int64_t row = r0 + rr;
      xs[rr][qq] = (row < rows && q0 + qq < l) ? (double)x[row * l + q0 + qq] : 0.0;
      const int qe = e >> 6, cc = e & 63;
      es[qe][cc] = (q0 + qe < l && c0 + cc < k) ? E[(int64_t)(q0 + qe) * lp + c0 + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int q = 0; q < 32; ++q) {
      double xv[4], ev[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        xv[a] = xs[ti * 4 + a][q];
        ev[a] = es[q][tj * 4 + a];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(xv[a], ev[b], acc[a][b]);
    }
  }
  float best[4], bsig[4];
  int bidx[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    best[b] = -1.0f;
    bsig[b] = 0.0f;
    bidx[b] = 0x7FFFFFFF;
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t row = r0 + ti * 4 + a;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = c0 + tj * 4 + b;
      if (row < rows && c < k) {
        const float v = (float)(colscale ? acc[a][b] * colscale[c] : acc[a][b]);
        out[row * k + c] = v;
        if (fabsf(v) > best[b]) {
          best[b] = fabsf(v);
          bsig[b] = v;
          bidx[b] = (int)row;
        }
      }
    }
  }
  if (!am_val) return;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    bvs[ti][tj * 4 + b] = best[b];
    bsg[ti][tj * 4 + b] = bsig[b];
    bis[ti][tj * 4 + b] = bidx[b];
  }
  __syncthreads();
  if (t < 64 && c0 + t < k) {
    float ba = -1.0f, val = 0.0f;
    int bi = 0x7FFFFFFF;
    for (int g = 0; g < 16; ++g)
      if (bvs[g][t] > ba) {
        ba = bvs[g][t];
        val = bsg[g][t];
        bi = bis[g][t];
      }
    am_val[blockIdx.x * k + c0 + t] = val;
    am_idx[blockIdx.x * k + c0 + t] = bi;
  }
}


template <int NC>
void chol_steps(double *C, double *F, int l, const double *aux, hipStream_t st) {
  for (int j0 = 0; j0 < l; j0 += kPiv) {
    const int below = l - std::min(j0 + kPiv, l);
    const unsigned grid = (unsigned)std::max<int64_t>(1, cdiv(below, kWT / 64));
    wchol_step_kernel<NC><<<grid, kWT, 0, st>>>(C, F, l, j0, aux);
  }
}

template <int NC>
void tri_steps(double *W, int l, double *V, double *beta, double *dg, double *eo, double *pbuf, hipStream_t st) {
  for (int j = -1; j <= l - 3 || j == -1; ++j) {
    const int below = l - (j + 2);
    const unsigned grid = (unsigned)std::max<int64_t>(1, cdiv(std::max(below, 0), kWT / 64));
    wtri_step_kernel<NC><<<grid, kWT, 0, st>>>(W, l, j, V, beta, dg, eo, pbuf);
  }
}

// The column count lp / 64 as a compile-time constant (lp a multiple of 64).
template <template <int> class Fn, typename... Args>
bool by_columns(int lp, Args... args) {
  switch (lp / 64) {
    case 2: Fn<2>::run(args...); return true;
    case 3: Fn<3>::run(args...); return true;
    case 4: Fn<4>::run(args...); return true;
    case 5: Fn<5>::run(args...); return true;
    case 6: Fn<6>::run(args...); return true;
    case 7: Fn<7>::run(args...); return true;
    case 8: Fn<8>::run(args...); return true;
  }
  return false;
}
template <int NC> struct CholSteps {
  static void run(double *C, double *F, int l, const double *aux, hipStream_t st) { chol_steps<NC>(C, F, l, aux, st); }
};
template <int NC> struct TriSteps {
  static void run(double *W, int l, double *V, double *beta, double *dg, double *eo, double *pbuf, hipStream_t st) {
    tri_steps<NC>(W, l, V, beta, dg, eo, pbuf, st);
  }
};

}  // namespace

namespace metis_wide {

size_t aux_doubles(int lp) { return (size_t)8 * lp + 64; }

metis_status_t wide_chol_inv(const double *g, int l, int lp, double *rinv, int *info, double *C, double *F,
                             double *aux, hipStream_t st) {
  if (l < 1 || l > kWideMax || lp < l || lp > kWideMax || lp % 64 || lp < 128) return METIS_ERR_UNSUPPORTED;
  const unsigned fill = (unsigned)cdiv((int64_t)lp * lp, kWT);
  wchol_init_kernel<<<fill, kWT, 0, st>>>(g, l, lp, C, aux);
  by_columns<CholSteps>(lp, C, F, l, (const double *)aux, st);
  wchol_finish_kernel<<<fill, kWT, 0, st>>>(F, l, lp, aux, rinv, info);
  return hipGetLastError() == hipSuccess ? METIS_OK : METIS_ERR_HIP;
}

metis_status_t wide_assemble(const float *x, int64_t rows, int l, int lp, int k, const double *evec,
                             const double *colscale, float *out, float *am_val, int *am_idx, hipStream_t st) {
  if (rows <= 0) return METIS_OK;
  wassemble_kernel<<<dim3((unsigned)cdiv(rows, 64), (unsigned)cdiv(k, 64)), kWT, 0, st>>>(x, rows, l, lp, k, evec,
                                                                                        colscale, out, am_val, am_idx);
  return hipGetLastError() == hipSuccess ? METIS_OK : METIS_ERR_HIP;
}

metis_status_t eigh_tridiag(int l, int lp, int k, const double *V, double *evec, double *sig_inv, float *S,
                            double *Dm, double *aux, hipStream_t st) {
  if (l < 1 || l > kWideMax || lp < l || lp > kWideMax || k < 1 || k > l || k > kWT) return METIS_ERR_UNSUPPORTED;
  double *dg = aux, *eo = aux + lp, *beta = aux + 2 * lp, *lam = aux + 5 * lp, *tn = aux + 6 * lp;
  weig_values_kernel<<<(unsigned)cdiv(k, kWT / 64), kWT, 0, st>>>(dg, eo, l, k, lam, tn);
  if (l <= kNarrow)
    neig_vectors_kernel<<<1, kWT, 0, st>>>(dg, eo, l, lp, k, lam, evec, sig_inv, S);
  else
    weig_vectors_kernel<<<1, kWT, 0, st>>>(dg, eo, l, lp, k, lam, evec, Dm, sig_inv, S);
  switch ((lp + 63) / 64) {
    case 1: launch_back<1>(evec, l, lp, k, V, beta, st); break;
    case 2: launch_back<2>(evec, l, lp, k, V, beta, st); break;
    case 3: launch_back<3>(evec, l, lp, k, V, beta, st); break;
    case 4: launch_back<4>(evec, l, lp, k, V, beta, st); break;
    case 5: launch_back<5>(evec, l, lp, k, V, beta, st); break;
    case 6: launch_back<6>(evec, l, lp, k, V, beta, st); break;
    case 7: launch_back<7>(evec, l, lp, k, V, beta, st); break;
    default: launch_back<8>(evec, l, lp, k, V, beta, st); break;
  }
  return hipGetLastError() == hipSuccess ? METIS_OK : METIS_ERR_HIP;
}

metis_status_t wide_eigh(const double *g, int l, int lp, int k, double *evec, double *sig_inv, float *S, double *W,
                         double *V, double *Dm, double *aux, hipStream_t st) {
  if (l < 1 || l > kWideMax || lp < l || lp > kWideMax || lp % 64 || lp < 128 || k < 1 || k > l || k > kWT)
    return METIS_ERR_UNSUPPORTED;
  double *dg = aux, *eo = aux + lp, *beta = aux + 2 * lp, *pbuf = aux + 3 * lp;
  const unsigned fill = (unsigned)cdiv((int64_t)lp * lp, kWT);
  wtri_init_kernel<<<fill, kWT, 0, st>>>(g, l, lp, W);
  by_columns<TriSteps>(lp, W, l, V, beta, dg, eo, pbuf, st);
  return eigh_tridiag(l, lp, k, V, evec, sig_inv, S, Dm, aux, st);
}

}  // namespace metis_wide
