// Host entry points of the wide-sketch (96 < l <= 512) small-matrix stages
// (wide.hip). All matrices are lp x lp fp64, row-major; lp <= kWideMax.
#pragma once
#include <stddef.h>

#include "metis_fp4.h"

namespace metis_wide {

constexpr int kWideMax = 512;

// Doubles of the small-vector scratch both calls take (aux).
size_t aux_doubles(int lp);

// rinv = R^-1 for G = R^T R (upper triangle of g read); a pivot at or below
// l 2^-52 max diag G is absent (zero row and column of R^-1, info = its
// 1-based index; info may be NULL). C, F: lp x lp scratch.
metis_status_t wide_chol_inv(const double *g, int l, int lp, double *rinv, int *info, double *C, double *F,
                             double *aux, hipStream_t st);

// The k largest eigenpairs of the symmetric g (upper triangle read):
// evec[row * lp + rank] (unit columns, descending eigenvalue, rows beyond l
// zero), sig_inv[rank] = 1 / sqrt(lambda) (0 for sqrt(lambda) at or below
// 2^-24 of the largest and for ranks >= k), S[rank < k] = sqrt(lambda).
// W, V, Dm: lp x lp scratch.
metis_status_t wide_eigh(const double *g, int l, int lp, int k, double *evec, double *sig_inv, float *S, double *W,
                         double *V, double *Dm, double *aux, hipStream_t st);

// The same eigenpairs from a tridiagonal reduction already made: T's
// diagonal in aux[0 .. l), its off-diagonal in aux[lp ..), the reflector
// scales beta_j in aux[2 lp ..), reflector j in V[j * lp + row] (G = H T H^T,
// H = H_0 ... H_{l-3}, H_j = I - beta_j v_j v_j^T). Dm: lp x lp scratch.
metis_status_t eigh_tridiag(int l, int lp, int k, const double *V, double *evec, double *sig_inv, float *S,
                            double *Dm, double *aux, hipStream_t st);

// out (rows x k, fp32) = x (rows x l fp32) E[:, :k] diag(colscale) (colscale
// may be NULL), fp64 sums; with am_val / am_idx (may be NULL), per tile of 64
// rows the argmax of |out[:, c]| (lowest row on ties) at [tile * k + c].
metis_status_t wide_assemble(const float *x, int64_t rows, int l, int lp, int k, const double *evec,
                             const double *colscale, float *out, float *am_val, int *am_idx, hipStream_t st);

}  // namespace metis_wide
