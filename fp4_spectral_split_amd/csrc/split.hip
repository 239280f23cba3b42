// metis_split: randomized spectral split A = U_k diag(S_k) V_k^T + R with
// block FP4 quantization of the parts.
//
// Method: SII open-source-week post on Metis §2.4 item 1 (dominant part +
// long-tail residual, decomposition in a low-dimensional space); "Metis:
// Training LLMs with FP4 Quantization", abstract (random projection / sparse
// random sampling). The steps are the randomized SVD of Halko, Martinsson &
// Tropp (SIAM Review 2011) Alg. 4.1 (range finder, no power iteration) and
// Alg. 5.1 (direct SVD):
//
//   pass 1 over A  sketch        Y = A Omega  (bf16 MFMA, fp32 accumulate;
//                                 split-K partials)       or Y = A[:, J]
//                  range         CholeskyQR2 on Y: fp64 Gram, one-workgroup
//                                 Cholesky + triangular inverse, Y R^-1, twice
//   pass 2 over A  projection    B^T = A^T Q  (Q as bf16 hi + lo: fp32-accurate)
//                  small SVD     eigen-decomposition of B B^T (fp64, l x l) in one
//                                 workgroup: Householder tridiagonalization,
//                                 multisection, twisted-factorization vectors
//                                 (l > 96: the multi-workgroup forms of wide.hip)
//                  assemble      U = Q E_k, S = sqrt(lambda_k), V = B^T E_k / S
//                  signs         largest-|entry| of each U column made positive
//                  factors       U^T, V^T block-quantized along their length
//   pass 3 over A  residual      R = A - U S V^T via bf16 hi/lo MFMA, then block
//                                 absmax, scale, E2M1 rounding and nibble packing
//                                 in both orientations from one LDS tile
//
// Every reduction runs in a fixed order (no atomics except the order-free
// integer max of NVFP4 tensor scales), so results are bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "wide.hpp"

using namespace metis;

namespace {

constexpr int kLpMax = 96;
constexpr int kSketchRS = 2;  // 16-row groups per wave in the sketch (a workgroup: 64 kSketchRS rows)
constexpr int kMaxPowerIterations = 16;  // Gaussian / sampled sketch width handled in LDS
constexpr int kThreads = 256;
// workgroups resident at once in the sketch and projection launches: two per
// CU (two waves per SIMD) on the 256 CUs
constexpr int64_t kSlots = 512;
constexpr int kGramRows = 64;      // rows per Gram chunk (narrow path)
constexpr int kGramThreads = 512;  // 8 waves: two per 16-row block
// assemble kernels: 16 rows per thread, at most 8 row groups (128 rows) per workgroup
constexpr int kAsmRows = 16;
constexpr int kAsmGroups = 8;
__host__ __device__ __forceinline__ int asm_groups(int k) { return kThreads / k < kAsmGroups ? kThreads / k : kAsmGroups; }
__host__ __device__ __forceinline__ int asm_chunk_rows(int k) { return kAsmRows * asm_groups(k); }

// ===================================================================== plan
struct SplitPlan {
  int64_t m, n;
  int l, lp, k, kp;
  int power;  // power iterations
  bool wide;  // l > kLpMax: global-memory forms of the small kernels
  int kind, fmt;
  int elem;  // bytes per input element
  // sketch
  int sk;
  int64_t sk_chunk;
  // gram over rows of Y (and Q1)
  int64_t gy_rows;
  int gy_parts;
  // projection
  int pk;
  int64_t pk_rows;
  // gram over rows of B^T
  int64_t gb_rows;
  int gb_parts;
  // assemble U argmax chunks
  int64_t am_rows;
  int am_parts;
  // workspace
  unsigned short *omt;   // lp x n bf16 (Omega^T, zero padded)
  float *ysk;            // sk x m x l
  float *y;              // m x l
  float *q1;             // m x l
  float *q;              // m x l
  unsigned short *qt;    // 2 x lp x m bf16 (hi, lo) transposed, zero padded rows
  float *btp;            // pk x n x l
  float *bt;             // n x l
  double *gpart;         // max(gy_parts, gb_parts) x lp x lp
  double *gram;          // lp x lp
  double *rinv;          // lp x lp
  double *evec;          // lp x lp
  double *sig_inv;       // lp (1/sigma, 0 for dropped)
  float *am_val;         // am_parts x k (value at argmax)
  int *am_idx;           // am_parts x k
  float *sign;           // k
  unsigned short *uhl;   // 2 x m x kp bf16 (U hi, lo)
  unsigned short *whl;   // 2 x n x kp bf16 ((V S) hi, lo)
  double *wa, *winv, *wg, *wv;  // lp x lp scratch of the global-memory (wide) forms
  double *waux;                 // small vectors of the wide forms
  uint32_t *amax;        // 8 words: NVFP4 tensor maxima (U^T, V^T, R)
  float *z1;             // n x l (power iterations: A^T Q after one R^-1)
  unsigned short *zt;    // 2 x lp x n bf16 (power iterations: orth(A^T Q)^T hi, lo)
  int *info_ws;          // 1 word
  size_t bytes;
};

// Split-K factor of a launch of `tiles` output tiles whose contraction takes
// `steps` steps of `step_bytes` per workgroup, each split writing a partial
// of `part_bytes` that the next kernel reads. The workgroups run in rounds of
// kSlots and a workgroup's time is its steps plus about two (its first loads
// and its stores), so the cost in bytes moved is rounds x (steps per
// workgroup + 2) x kSlots x step_bytes + 2 x factor x part_bytes; the least
// cost wins, the smallest factor on a tie.
int64_t pick_split(int64_t tiles, int64_t steps, int64_t step_bytes, int64_t part_bytes) {
  int64_t best = 1, best_cost = INT64_MAX;
  for (int64_t f = 1; f <= std::min<int64_t>(steps, 64); ++f) {
    const int64_t cost = cdiv(tiles * f, kSlots) * (cdiv(steps, f) + 2) * kSlots * step_bytes + 2 * f * part_bytes;
    if (cost < best_cost) best = f, best_cost = cost;
  }
  return best;
}

int64_t pick_rows_per_part(int64_t rows, int64_t want_parts, int64_t quantum) {
  int64_t per = round_up(cdiv(rows, std::max<int64_t>(1, want_parts)), quantum);
  return std::max<int64_t>(per, quantum);
}

SplitPlan make_plan(int64_t m, int64_t n, int l, int k, int kind, int fmt, int elem, void *ws, int q = 0) {
  SplitPlan p;
  p.m = m; p.n = n; p.l = l; p.k = k; p.kind = kind; p.fmt = fmt; p.elem = elem; p.power = q;
  p.wide = l > kLpMax;
  p.lp = (int)round_up(l, p.wide ? 64 : 16);
  p.kp = (int)round_up(k, 32);
  // sketch: 128-row tiles of 128-column steps, split-K as pick_split finds
  const int64_t l_tiles = cdiv(p.lp, kLpMax);
  if (kind == METIS_OMEGA_GAUSSIAN || q > 0) {
    const int64_t want = pick_split(cdiv(m, 128) * l_tiles, cdiv(n, 128), 128 * 128 * elem, m * p.lp * 4);
    p.sk_chunk = round_up(cdiv(n, want), 128);
    p.sk = (int)cdiv(n, p.sk_chunk);
  } else {
    p.sk = 1;
    p.sk_chunk = n;
  }
  // narrow Grams: one partial per 128-row chunk; wide Grams: 16 row ranges
  p.gy_rows = p.wide ? pick_rows_per_part(m, 16, 32) : kGramRows;
  p.gy_parts = (int)cdiv(m, p.gy_rows);
  // projection: 128-column tiles of 64-row steps, split the same way
  const int64_t wantp = pick_split(cdiv(n, 128) * l_tiles, cdiv(m, 64), 64 * 128 * elem, n * p.lp * 4);
  p.pk_rows = round_up(cdiv(m, wantp), 64);
  p.pk = (int)cdiv(m, p.pk_rows);
  p.gb_rows = p.wide ? pick_rows_per_part(n, 16, 32) : kGramRows;
  p.gb_parts = (int)cdiv(n, p.gb_rows);
  p.am_rows = p.wide ? 64 : asm_chunk_rows(k);  // rows per argmax partial of the assemble kernels
  p.am_parts = (int)cdiv(m, p.am_rows);

  metis_host::Carver c(ws);
  p.omt = c.take<unsigned short>((size_t)p.lp * n);
  p.ysk = c.take<float>((size_t)p.sk * m * l);
  p.y = c.take<float>((size_t)m * l);
  p.q1 = c.take<float>((size_t)m * l);
  p.q = c.take<float>((size_t)m * l);
  p.qt = c.take<unsigned short>((size_t)2 * p.lp * m);
  p.btp = c.take<float>((size_t)p.pk * n * l);
  p.bt = c.take<float>((size_t)n * l);
  p.gpart = c.take<double>((size_t)std::max(p.gy_parts, p.gb_parts) * p.lp * p.lp);
  p.gram = c.take<double>((size_t)p.lp * p.lp);
  p.rinv = c.take<double>((size_t)p.lp * p.lp);
  p.evec = c.take<double>((size_t)p.lp * p.lp);
  p.sig_inv = c.take<double>((size_t)p.lp);
  p.am_val = c.take<float>((size_t)p.am_parts * k);
  p.am_idx = c.take<int>((size_t)p.am_parts * k);
  p.sign = c.take<float>((size_t)k);
  p.uhl = c.take<unsigned short>((size_t)2 * m * p.kp);
  p.whl = c.take<unsigned short>((size_t)2 * n * p.kp);
  p.wa = c.take<double>((size_t)p.lp * p.lp);
  p.winv = c.take<double>((size_t)p.lp * p.lp);
  p.wg = c.take<double>((size_t)p.lp * p.lp);
  p.wv = c.take<double>((size_t)p.lp * p.lp);
  p.waux = c.take<double>(metis_wide::aux_doubles(p.lp));
  p.amax = c.take<uint32_t>(8);
  p.info_ws = c.take<int>(1);
  p.z1 = c.take<float>(q > 0 ? (size_t)n * l : 0);
  p.zt = c.take<unsigned short>(q > 0 ? (size_t)2 * p.lp * n : 0);
  p.bytes = c.bytes();
  return p;
}

// ============================================================ small kernels
__global__ void fill_u32(uint32_t *p, uint32_t v, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}

// Omega (n x l bf16, row-major) -> Omega^T (lp x n), rows l..lp-1 zero.
// 64 rows of Omega per workgroup through an LDS tile: the rows are read as
// one contiguous block and the columns written contiguously.
constexpr int kOtRows = 64;
__global__ void __launch_bounds__(256) omega_transpose_kernel(const unsigned short *__restrict__ om, int64_t n, int l,
                                                              int lp, unsigned short *__restrict__ omt) {
  __shared__ unsigned short tile[metis_wide::kWideMax][kOtRows + 2];  // l <= 512 columns
  const int t = threadIdx.x;
  const int64_t j0 = (int64_t)blockIdx.x * kOtRows;
  const int rows = (int)std::min<int64_t>(kOtRows, n - j0);
  const unsigned short *src = om + j0 * l;
  for (int e = t; e < rows * l; e += 256) tile[e % l][e / l] = src[e];
  __syncthreads();
  for (int e = t; e < lp * kOtRows; e += 256) {
    const int c = e / kOtRows, jj = e % kOtRows;
    if (jj < rows) omt[(int64_t)c * n + j0 + jj] = c < l ? tile[c][jj] : (unsigned short)0;
  }
}

// ================================================================== sketch
// ysk[s] = A[:, chunk s] * Omega[chunk s, :]. 4 waves x 32 rows; the Omega^T
// chunk (lp x 128) is staged in LDS and shared by the waves. A step is four
// 32-column MFMA slots; lane (r, g) holds elements 8g .. 8g + 7 of each slot
// of its row, so one load instruction reads 64 contiguous bytes of each of
// its 16 rows (a lane reading 64 contiguous bytes of one slot-permuted row
// took 5-20 % longer). The next step's A elements and Omega^T pieces are
// loaded into registers while the current step is multiplied.
// HL: the right-hand factor is an fp32 matrix carried as bf16 hi + lo
// (omt holds its hi rows 0 .. lp - 1, then its lo rows), both multiplied, so
// the product is fp32-accurate (the power iterations' Y = A Z).
template <typename T, bool HL = false, int RS = kSketchRS, int NC = 0>
__global__ void __launch_bounds__(kThreads) sketch_kernel(const T *__restrict__ A, int64_t m, int64_t n, int64_t lda,
                                                          const unsigned short *__restrict__ omt, int l, int lp,
                                                          int64_t chunk, float *__restrict__ ysk) {
  // blockIdx.z selects a tile of kLpMax sketch columns starting at l0
  const int l0 = blockIdx.z * kLpMax;
  const int lt = min(kLpMax, lp - l0);
  constexpr int KS = 128;
  constexpr int NT = (sizeof(T) == 4) ? 3 : 1;  // bf16 terms per element (fp32 = hi + mid + lo)
  constexpr int AV = 32 * (int)sizeof(T) / 16;   // 16-byte pieces of A per lane and row
  constexpr int OPR = (kLpMax * (KS / 8) + kThreads - 1) / kThreads;  // Omega^T pieces per thread
  constexpr int NH = HL ? 2 : 1;  // bf16 parts of the right-hand factor
  __shared__ __attribute__((aligned(16))) unsigned short lds[NH][kLpMax][KS + 8];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (64 * RS) + wave * (16 * RS);
  const int s = blockIdx.y;
  const int64_t c_beg = (int64_t)s * chunk;
  const int64_t c_end = std::min<int64_t>(n, c_beg + chunk);
  // NC > 0: the launch has exactly NC 16-column tiles (no runtime test, so
  // the accumulators never leave the MFMA registers)
  constexpr int NCM = NC ? NC : kLpMax / 16;
  const int nct = NC ? NC : lt >> 4;
  floatx4 acc[RS][NCM];
#pragma unroll
  for (int a = 0; a < RS; ++a)
#pragma unroll
    for (int b = 0; b < NCM; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Every load takes a clamped, valid address and none sits in a branch, so
  // the waits for a step's data stay counted while the next step's loads
  // are in flight: rows past m only feed rows of ysk that are not stored;
  // A's columns past the chunk are zeroed when the step is taken (n and the
  // chunk ends are multiples of 32, so a 32-column slot is all in or all
  // out), which also cancels the clamped Omega columns they meet; Omega^T
  // rows past lt go to LDS rows that no MFMA reads.
  static_assert(OPR * kThreads == kLpMax * (KS / 8), "Omega^T pieces fill the LDS rows exactly");
  // one step's loads, returned by value (vector values stay in registers)
  struct Step {
    intx4 a[RS][AV];
    intx4 o[NH][OPR];
  };
  auto load = [&](int64_t c0) {
    Step st;
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      const int64_t row = min(row0 + rs * 16 + r16, m - 1);
      const T *arow = A + row * lda;
#pragma unroll
      for (int j = 0; j < AV; ++j) {
        const int64_t cc = min(c0 + (j / (AV / 4)) * 32 + g * 8 + (j % (AV / 4)) * (16 / (int)sizeof(T)),
                               n - 16 / (int)sizeof(T));
        st.a[rs][j] = *(const intx4 *)(arow + cc);
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int p = 0; p < OPR; ++p) {
        const int idx = t + kThreads * p;
        const int rr = min(idx / (KS / 8), lt - 1), q = idx % (KS / 8);
        const int64_t cc = min(c0 + q * 8, n - 8);
        st.o[h][p] = *(const intx4 *)(omt + ((int64_t)h * lp + l0 + rr) * n + cc);
      }
    return st;
  };

  intx4 ca[RS][AV];
  Step nx = load(c_beg < c_end ? c_beg : 0);
  for (int64_t c0 = c_beg; c0 < c_end; c0 += KS) {
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int p = 0; p < OPR; ++p) {
        const int idx = t + kThreads * p;
        *(intx4 *)&lds[h][idx / (KS / 8)][(idx % (KS / 8)) * 8] = nx.o[h][p];
      }
#pragma unroll
    for (int rs = 0; rs < RS; ++rs)
#pragma unroll
      for (int j = 0; j < AV; ++j) ca[rs][j] = nx.a[rs][j] & (c0 + (j / (AV / 4)) * 32 < c_end ? -1 : 0);
    // the next step's loads (the last step reloads itself, from cache) are
    // in flight while this step is multiplied
    nx = load(c0 + KS < c_end ? c0 + KS : c0);
    __syncthreads();
    ushortx8 a[RS][4][NT];
#pragma unroll
    for (int rs = 0; rs < RS; ++rs) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[rs][j][0] = __builtin_bit_cast(ushortx8, ca[rs][j]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 v0 = __builtin_bit_cast(float4, ca[rs][2 * j]);
          const float4 v1 = __builtin_bit_cast(float4, ca[rs][2 * j + 1]);
          const float xs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // exact three-way split: x = hi + mid + lo, each a bf16 value
            const unsigned short hi = f32_to_bf16(xs[e]);
            const float r1 = xs[e] - bf16_to_f32(hi);
            const unsigned short mid = f32_to_bf16(r1);
            const unsigned short lo = f32_to_bf16(r1 - bf16_to_f32(mid));
            a[rs][j][0][e] = hi;
            a[rs][j][NT > 1 ? 1 : 0][e] = mid;
            a[rs][j][NT > 2 ? 2 : 0][e] = lo;
          }
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCM; ++ct) {
      if (NC || ct < nct) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const ushortx8 b = *(const ushortx8 *)&lds[h][ct * 16 + r16][j * 32 + g * 8];
#pragma unroll
            for (int rs = 0; rs < RS; ++rs)
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) acc[rs][ct] = mfma16_bf16(a[rs][j][tt], b, acc[rs][ct]);
          }
      }
    }
  }
  float *out = ysk + (int64_t)s * m * l;
#pragma unroll
  for (int rs = 0; rs < RS; ++rs)
#pragma unroll
    for (int ct = 0; ct < NCM; ++ct) {
      if (NC || ct < nct) {
        const int col = l0 + ct * 16 + r16;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t row = row0 + rs * 16 + g * 4 + t;
          if (row < m && col < l) out[row * l + col] = acc[rs][ct][t];
        }
      }
    }
}

// Y[:, c] = A[:, J[c]] (exact). Ids outside [0, n) read as zero columns.
template <typename T>
__global__ void gather_kernel(const T *__restrict__ A, int64_t m, int64_t n, int64_t lda, const int *__restrict__ J,
                              int l, float *__restrict__ y) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (idx >= m * l) return;
  const int64_t r = idx / l;
  const int c = (int)(idx - r * l);
  const int j = J[c];
  y[idx] = (j >= 0 && j < n) ? load_f32(A + r * lda + j) : 0.0f;
}


// sum of `parts` values spaced `stride` apart, in a fixed order (four
// interleaved partial sums so the loads issue together)
__device__ __forceinline__ float sum_parts(const float *p, int parts, int64_t stride) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int q = 0;
  for (; q + 4 <= parts; q += 4) {
    s0 += p[q * stride];
    s1 += p[(q + 1) * stride];
    s2 += p[(q + 2) * stride];
    s3 += p[(q + 3) * stride];
  }
  for (; q < parts; ++q) s0 += p[q * stride];
  return (s0 + s1) + (s2 + s3);
}

// ==================================================================== gram
typedef double doublex4 __attribute__((ext_vector_type(4)));

// fp64 MFMA 16x16x4: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
// acc[i] holds C[l / 16 + 4 i][l % 16].
__device__ __forceinline__ doublex4 mfma16_f64(double a, double b, doublex4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// One 64-row chunk of a tall matrix X (rows x l, fp32, lp = l rounded up to 16):
//   rinv == nullptr: X = sum of `parts` slabs of xin (fixed order);
//   rinv != nullptr: X = xin R^-1 with fp64 products and sums (fp64 MFMA),
//                    rounded to fp32 (R^-1 upper triangular, lp x lp).
// X goes to xout (if given), to xt as bf16 hi/lo transposed (2 x lp x rows,
// if given), and the fp64 Gram X^T X of the chunk (upper 16 x 16 tiles) to
// gpart[chunk] (lp x lp, if given). Eight waves; the chunk sits in LDS. The
// two waves of a 16-row block share its column tiles of xin R^-1 (tile J
// reads columns below 16 (J + 1), so the costs differ; the tiles are dealt
// from the last in the order 0 1 1 0 0 1 1 0 ..., which evens them out) and
// write them to a second LDS copy; then each wave accumulates Gram tiles over
// the chunk's rows, 4 rows per MFMA. The fp64 matrix cores bound the kernel,
// so a chunk is kept short to spread a Gram over many workgroups.

__host__ __device__ constexpr int gram_ys_stride(int lp) { return lp + 4; }                  // (lp + 4) / 4 odd
__host__ __device__ constexpr int gram_rl_stride(int lp) { return lp % 32 == 16 ? lp : lp + 16; }  // 16 mod 32

// Rows [row0, row0 + kGramRows) of the sum of `parts` slabs of xin (row
// stride l, slab stride part_stride) into Ys (row stride S), summed in slab
// order; columns l .. lp - 1 and rows past `rows` are zero. For l % 4 == 0
// each thread loads float4s and keeps the loads of four slabs in flight
// together, so the chunk arrives in a few memory round trips.
__device__ __forceinline__ void gram_load_chunk(float *Ys, int S, const float *__restrict__ xin, int parts,
                                                int64_t part_stride, int64_t row0, int64_t rows, int l, int lp) {
  const int t = threadIdx.x;
  const int nrows = (int)std::min<int64_t>(kGramRows, rows - row0);
  if ((l & 3) == 0) {
    constexpr int NV = kGramRows * kLpMax / 4 / kGramThreads;
    const int nv = nrows * l / 4;
    const float4 *src = (const float4 *)(xin + row0 * l);
    const int64_t ps4 = part_stride / 4;
    const float4 z = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float4 acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = z;
    int q = 0;
    for (; q + 4 <= parts; q += 4) {
      float4 x[4][NV];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int f = t + i * kGramThreads;
          x[u][i] = f < nv ? src[(q + u) * ps4 + f] : z;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          acc[i].x += x[u][i].x;
          acc[i].y += x[u][i].y;
          acc[i].z += x[u][i].z;
          acc[i].w += x[u][i].w;
        }
    }
    for (; q < parts; ++q) {
      float4 x[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int f = t + i * kGramThreads;
        x[i] = f < nv ? src[q * ps4 + f] : z;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        acc[i].x += x[i].x;
        acc[i].y += x[i].y;
        acc[i].z += x[i].z;
        acc[i].w += x[i].w;
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int f = t + i * kGramThreads;
      if (f < nv) {
        const int r = (4 * f) / l, c = 4 * f - r * l;
        *(float4 *)(Ys + r * S + c) = acc[i];
      }
    }
    if (nrows < kGramRows || l < lp)
      for (int idx = t; idx < kGramRows * lp; idx += kGramThreads) {
        const int r = idx / lp, c = idx - (idx / lp) * lp;
        if (r >= nrows || c >= l) Ys[r * S + c] = 0.0f;
      }
  } else {
    for (int idx = t; idx < kGramRows * lp; idx += kGramThreads) {
      const int r = idx / lp, c = idx - (idx / lp) * lp;
      Ys[r * S + c] = (r < nrows && c < l) ? sum_parts(xin + (row0 + r) * l + c, parts, part_stride) : 0.0f;
    }
  }
}

__global__ void __launch_bounds__(kGramThreads)
    gram_kernel(const float *__restrict__ xin, int parts, int64_t part_stride, int64_t rows, int l, int lp,
                const double *__restrict__ rinv, float *__restrict__ xout, unsigned short *__restrict__ xt,
                double *__restrict__ gpart) {
  __shared__ __attribute__((aligned(16))) float Ys[kGramRows * (kLpMax + 4)];
  __shared__ __attribute__((aligned(16))) float Xs[kGramRows * (kLpMax + 4)];
  __shared__ double Rl[kLpMax * (kLpMax + 16)];
  static_assert(kGramRows == 64 && kGramThreads == 512, "four 16-row blocks, two waves each");
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, lr = lane & 15, lk = lane >> 4;
  const int S = gram_ys_stride(lp), RS = gram_rl_stride(lp), T = lp >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * kGramRows;
  gram_load_chunk(Ys, S, xin, parts, part_stride, row0, rows, l, lp);
  if (rinv) {
    // R^-1 in pairs of columns, every load of the thread in flight at once
    constexpr int NR = kLpMax * kLpMax / 2 / kGramThreads;
    const double2 *src = (const double2 *)rinv;
    const int nr = lp * lp / 2;
    double2 v[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = t + i * kGramThreads;
      v[i] = f < nr ? src[f] : make_double2(0.0, 0.0);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int f = t + i * kGramThreads;
      if (f < nr) {
        const int r = (2 * f) / lp, c = 2 * f - r * lp;
        Rl[r * RS + c] = v[i].x;
        Rl[r * RS + c + 1] = v[i].y;
      }
    }
  }
  __syncthreads();
  const float *X = Ys;
  if (rinv) {
    const int rb = 16 * (wave & 3), half = wave >> 2;
    for (int J = T - 1; J >= 0; --J) {
      const int d = (T - 1 - J) & 3;
      if ((d == 1 || d == 2) != (half == 1)) continue;
      doublex4 acc = {0.0, 0.0, 0.0, 0.0};
      for (int s4 = 0; s4 < 4 * (J + 1); ++s4) {
        const double a = (double)Ys[(rb + lr) * S + 4 * s4 + lk];
        const double b = Rl[(4 * s4 + lk) * RS + 16 * J + lr];
        acc = mfma16_f64(a, b, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Xs[(rb + lk + 4 * i) * S + 16 * J + lr] = (float)acc[i];
    }
    __syncthreads();
    X = Xs;
  }
  if (xout)
    for (int idx = t; idx < kGramRows * l; idx += kGramThreads) {
      const int r = idx / l, c = idx - (idx / l) * l;
      if (row0 + r < rows) xout[(row0 + r) * l + c] = X[r * S + c];
    }
  if (xt) {
    // 8 consecutive rows of one column per thread (16-byte stores)
    for (int idx = t; idx < lp * (kGramRows / 8); idx += kGramThreads) {
      const int c = idx / (kGramRows / 8), q = idx - c * (kGramRows / 8);
      if (row0 + q * 8 >= rows) continue;
      ushortx8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        unsigned short h, w;
        split_bf16(X[(q * 8 + e) * S + c], h, w);
        hi[e] = h;
        lo[e] = w;
      }
      *(ushortx8 *)(xt + (int64_t)c * rows + row0 + q * 8) = hi;
      *(ushortx8 *)(xt + ((int64_t)lp + c) * rows + row0 + q * 8) = lo;
    }
  }
  if (gpart) {
    double *g = gpart + (int64_t)blockIdx.x * lp * lp;
    const int ntiles = T * (T + 1) / 2;
    for (int tile = wave; tile < ntiles; tile += kGramThreads / 64) {
      int I = 0, rem = tile;  // tile -> (I, J), I <= J, row-major over the upper triangle
      while (rem >= T - I) {
        rem -= T - I;
        ++I;
      }
      const int J = I + rem;
      doublex4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
      for (int r = 0; r < kGramRows; r += 4) {
        const double a = (double)X[(r + lk) * S + 16 * I + lr];
        const double b = (double)X[(r + lk) * S + 16 * J + lr];
        acc = mfma16_f64(a, b, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) g[(16 * I + lk + 4 * i) * lp + 16 * J + lr] = acc[i];
    }
  }
}

// G = sum over parts of gpart (upper triangle is what the consumers read).
// Eight lanes per element, lane j summing parts j, j + 8, ...; the fixed DPP
// combine keeps the result independent of scheduling.
__global__ void __launch_bounds__(256)
    gram_reduce_kernel(const double *__restrict__ gpart, int parts, int lp2, double *__restrict__ g) {
  const int e = blockIdx.x * 32 + (threadIdx.x >> 3), j = threadIdx.x & 7;
  double s = 0.0;
  if (e < lp2) {
    // parts j, j + 8, ... in order, eight loads in flight per step
    int q = j;
    for (; q + 56 < parts; q += 64) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = gpart[(int64_t)(q + 8 * u) * lp2 + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; q < parts; q += 8) s += gpart[(int64_t)q * lp2 + e];
  }
  s = group8_sum(s);
  if (e < lp2 && j == 0) g[e] = s;
}

// ========================================================= Cholesky + inverse
// The factorization for l <= kLpMax as one elimination on [G | I]: step j
// subtracts m_p = G'[j][p] / d_j times row j from every later row p, on the
// upper part of the trailing matrix G' and on the block L^-1 that starts as
// I. After the last step the pivots d_j are those of G = L D L^T and the
// block holds L^-1, so R = D^1/2 L^T and R^-1 = L^-T D^-1/2. Absent pivots
// (d_j <= tol) get m_p = 0 and a zero row and column of R^-1.
// The steps are taken in panels of 16 pivots (blocked Gauss-Jordan):
//  - panel phase, wave 0 alone and without barriers: the panel's 16 rows sit
//    in registers (lane y holds columns y and y + 64 of the row laid out as
//    [L^-1 columns 0 .. j0 + 15 | G' columns j0 ..]) and are eliminated among
//    themselves; a step's multipliers are the pivot row's own entries at the
//    later rows' columns (the trailing matrix is symmetric), read from the
//    lanes that hold them;
//  - trailing phase, all four waves: every row p below the panel loses
//    sum_j m_pj row_j over the panel's final rows, m_pj = row_j[p] / d_j,
//    which is what the panel's 16 single steps would subtract from it.
// Each published row is final; the lower part of G' takes values that are
// never read. Rows and columns in [l, lpad) are zero: absent pivots.
constexpr int kCholThreads = 256;
constexpr int kCholPanel = 16;

__device__ __forceinline__ double recip_f64(double d) {
  double r = __builtin_amdgcn_rcp(d);  // hardware estimate, refined by Newton steps
  r = fma(r, fma(-d, r, 1.0), r);
  return fma(r, fma(-d, r, 1.0), r);
}

__global__ void __launch_bounds__(kCholThreads)
    chol_small_kernel(const double *__restrict__ g, int l, int lp, double *__restrict__ out, int *info) {
  // published rows of G' (upper part meaningful) and of L^-1, one array so
  // a lane can address either by an offset from its start
  __shared__ double CGL[2][kLpMax][kLpMax + 1];
  auto &CG = CGL[0];
  auto &CL = CGL[1];
  __shared__ double rs[kLpMax];               // d_j^-1/2, 0 for an absent pivot
  __shared__ double dinv[kLpMax];             // 1 / d_j, 0 for an absent pivot
  __shared__ int dead[kLpMax];
  __shared__ double tol_s;
  const int t = threadIdx.x;
  {
    // upper triangle of G (zeros elsewhere, also beyond l), all of a
    // thread's loads in flight together; CL = I
    constexpr int PER = (kLpMax * kLpMax + kCholThreads - 1) / kCholThreads;
    double v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + u * kCholThreads, p = e / kLpMax, x = e - p * kLpMax;
      v[u] = (e < kLpMax * kLpMax && p < l && x < l && x >= p) ? g[p * lp + x] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + u * kCholThreads, p = e / kLpMax, x = e - p * kLpMax;
      if (e < kLpMax * kLpMax) {
        CG[p][x] = v[u];
        CL[p][x] = p == x ? 1.0 : 0.0;
      }
    }
    {
      // the second CholeskyQR pass sees G = I + E with E tiny: then
      // R = I + F with F = triu(E), diag halved, and R^-1 = I - F up to
      // O(E^2) (below 1e-10 here), with no elimination at all. A dead
      // column of the first pass leaves E_jj = -1 and takes the full path.
      __shared__ double emax_w[kCholThreads / 64];
      double em = 0.0;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = t + u * kCholThreads, p = e / kLpMax, x = e - p * kLpMax;
        if (e < kLpMax * kLpMax && p < l && x < l && x >= p) em = fmax(em, fabs(v[u] - (x == p ? 1.0 : 0.0)));
      }
      em = wave_max(em);
      if ((t & 63) == 0) emax_w[t >> 6] = em;
      __syncthreads();
      double emax = 0.0;
#pragma unroll
      for (int w = 0; w < kCholThreads / 64; ++w) emax = fmax(emax, emax_w[w]);
      if (emax < 1e-5) {
        for (int e = t; e < lp * lp; e += kCholThreads) {
          const int i = e / lp, c = e - (e / lp) * lp;
          double r = 0.0;
          if (c < l && i <= c) r = i == c ? 1.0 - 0.5 * (CG[i][i] - 1.0) : -CG[i][c];
          out[e] = r;
        }
        if (t == 0 && info) *info = 0;
        return;
      }
    }
  }
  if (t < 64) {
    double md = 0.0;
    for (int i = t; i < l; i += 64) md = fmax(md, CG[i][i]);
    md = wave_max(md);
    if (t == 0) tol_s = (double)l * 2.220446049250313e-16 * md;
  }
  constexpr int PB = kCholPanel;
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lpad = (l + PB - 1) / PB * PB;
  __syncthreads();
  const double tol = tol_s;
  // Every LDS access below is unconditional, its address selected per lane
  // (a lane with no element uses the pad column kLpMax of CG, never read as
  // data), so no branch separates the accesses and they stay in flight
  // together.
  for (int j0 = 0; j0 < lpad; j0 += PB) {
    if (wave == 0) {
      // unified column y: L^-1 column y for y < j0 + PB, else G' column y - PB
      double *ad[2];
      bool ok[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int y = lane + 64 * s;
        ok[s] = y - PB < kLpMax;
        ad[s] = y < j0 + PB ? &CL[j0][y] : &CG[j0][ok[s] ? y - PB : kLpMax];
      }
      double pr[PB][2];
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const double v = ad[s][q * (kLpMax + 1)];
          pr[q][s] = ok[s] ? v : 0.0;
        }
#pragma unroll
      for (int jj = 0; jj < PB; ++jj) {
        const int yd = j0 + jj + PB;  // d_j = G'[j][j]
        const double d = readlane_f64(yd < 64 ? pr[jj][0] : pr[jj][1], yd & 63);
        const double id = d > tol ? recip_f64(d) : 0.0;
        dinv[j0 + jj] = id;  // the same value from every lane
#pragma unroll
        for (int q = jj + 1; q < PB; ++q) {
          const int yq = j0 + q + PB;  // G'[j][j0 + q]
          const double m = readlane_f64(yq < 64 ? pr[jj][0] : pr[jj][1], yq & 63) * id;
          pr[q][0] = fma(-m, pr[jj][0], pr[q][0]);
          pr[q][1] = fma(-m, pr[jj][1], pr[q][1]);
        }
      }
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int s = 0; s < 2; ++s) ad[s][q * (kLpMax + 1)] = pr[q][s];
    }
    __syncthreads();
    const int p0 = j0 + PB;
    if (p0 < lpad) {
      // unified column y: L^-1 column y for y < p0, else G' column y
      int off[2];
      bool ok[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int y = lane + 64 * s;
        ok[s] = y < lpad;
        off[s] = y < p0 ? kLpMax * (kLpMax + 1) + y : (ok[s] ? y : kLpMax);
      }
      double *const base = &CGL[0][0][0];
      double pv[PB][2], idv[PB];
#pragma unroll
      for (int jj = 0; jj < PB; ++jj) {
        idv[jj] = dinv[j0 + jj];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const double v = base[off[s] + (j0 + jj) * (kLpMax + 1)];
          pv[jj][s] = ok[s] ? v : 0.0;
        }
      }
      for (int p = p0 + wave; p < lpad; p += kCholThreads / 64) {
        double acc[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) acc[s] = base[off[s] + p * (kLpMax + 1)];
#pragma unroll
        for (int jj = 0; jj < PB; ++jj) {
          const double m = CG[j0 + jj][p] * idv[jj];
          acc[0] = fma(-m, pv[jj][0], acc[0]);
          acc[1] = fma(-m, pv[jj][1], acc[1]);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) base[off[s] + p * (kLpMax + 1)] = acc[s];
      }
    }
    __syncthreads();
  }
  // pivots d_j sit on the diagonal of the published rows
  for (int j = t; j < l; j += kCholThreads) {
    const double d = CG[j][j];
    const bool alive = d > tol;
    rs[j] = alive ? 1.0 / sqrt(d) : 0.0;
    dead[j] = !alive;
  }
  __syncthreads();
  // R^-1[i][c] = L^-1[c][i] * d_c^-1/2 for i <= c < l; zero elsewhere
  for (int e = t; e < lp * lp; e += kCholThreads) {
    const int i = e / lp, c = e - (e / lp) * lp;
    double r = 0.0;
    if (c < l && i <= c) r = CL[c][i] * rs[c];
    out[e] = r;
  }
  if (t == 0 && info) {
    int first = 0;
    for (int j = l - 1; j >= 0; --j)
      if (dead[j]) first = j + 1;
    *info = first;
  }
}

// ----------------------------------------------- wide-sketch helpers (l > 96)
// x = sum over parts (fixed order); rows x l elements.
// x = sum over n_parts slabs (slab order), four elements per thread with
// the loads of eight slabs in flight: the projection's partials are summed
// by the whole GPU before their Gram (count % 4 == 0, 16-byte aligned).
__global__ void __launch_bounds__(256)
    sum_parts4_kernel(const float *__restrict__ parts, int n_parts, int64_t stride, int64_t count,
                      float *__restrict__ x) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  int q = 0;
  for (; q + 8 <= n_parts; q += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const float4 *)(parts + (int64_t)(q + u) * stride + i);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  for (; q < n_parts; ++q) {
    const float4 v = *(const float4 *)(parts + (int64_t)q * stride + i);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *(float4 *)(x + i) = acc;
}

__global__ void sum_parts_kernel(const float *__restrict__ parts, int n_parts, int64_t stride, int64_t count,
                                 float *__restrict__ x) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= count) return;
  x[i] = sum_parts(parts + i, n_parts, stride);
}

// Partial Gram tile over one chunk of rows: gpart[chunk] (lp x lp) rows
// [64 ti, +64) x columns [64 tj, +64), fp64; thread owns a 4 x 4 block.
__global__ void __launch_bounds__(kThreads)
    gram_tile_kernel(const float *__restrict__ x, int64_t rows, int l, int lp, int64_t rows_per_chunk,
                     double *__restrict__ gpart) {
  __shared__ float xi[32][65], xj[32][65];
  const int t = threadIdx.x;
  const int ti = blockIdx.y, tj = blockIdx.z;
  const int bi = t >> 4, bj = t & 15;
  const int64_t r_beg = blockIdx.x * rows_per_chunk;
  const int64_t r_end = std::min<int64_t>(rows, r_beg + rows_per_chunk);
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int64_t r0 = r_beg; r0 < r_end; r0 += 32) {
    __syncthreads();
    for (int idx = t; idx < 32 * 64; idx += kThreads) {
      const int rr = idx >> 6, c = idx & 63;
      const int64_t row = r0 + rr;
      const int ci = ti * 64 + c, cj = tj * 64 + c;
      xi[rr][c] = (row < r_end && ci < l) ? x[row * l + ci] : 0.0f;
      xj[rr][c] = (row < r_end && cj < l) ? x[row * l + cj] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 32; ++rr) {
      double vi[4], vj[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        vi[a] = xi[rr][bi * 4 + a];
        vj[a] = xj[rr][bj * 4 + a];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += vi[a] * vj[b];
    }
  }
  double *g = gpart + (int64_t)blockIdx.x * lp * lp;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) g[(ti * 64 + bi * 4 + a) * lp + tj * 64 + bj * 4 + b] = acc[a][b];
}

// xout = xin R^-1 (fp64 accumulate, fp32 out) on 64 x 64 output tiles;
// optionally also bf16 hi/lo of xout transposed into xt (2 x lp x rows).
__global__ void __launch_bounds__(kThreads)
    apply_rinv_kernel(const float *__restrict__ xin, int64_t rows, int l, int lp, const double *__restrict__ rinv,
                      float *__restrict__ xout, unsigned short *__restrict__ xt) {
  __shared__ float xs[64][65];
  __shared__ double rs[64][65];
  const int t = threadIdx.x;
  const int64_t r0 = blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int bi = t >> 4, bj = t & 15;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int k0 = 0; k0 <= c0; k0 += 64) {  // R^-1 is upper triangular
    __syncthreads();
    for (int idx = t; idx < 64 * 64; idx += kThreads) {
      const int rr = idx >> 6, c = idx & 63;
      xs[rr][c] = (r0 + rr < rows && k0 + c < l) ? xin[(r0 + rr) * l + k0 + c] : 0.0f;
      rs[rr][c] = rinv[(int64_t)(k0 + rr) * lp + c0 + c];
    }
    __syncthreads();
    for (int q = 0; q < 64; ++q) {
      double vx[4], vr[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        vx[a] = xs[bi * 4 + a][q];
        vr[a] = rs[q][bj * 4 + a];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += vx[a] * vr[b];
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t r = r0 + bi * 4 + a;
    if (r >= rows) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = c0 + bj * 4 + b;
      const float v = (float)acc[a][b];
      if (xout && c < l) xout[r * l + c] = v;
      if (xt) {
        unsigned short hi, lo;
        split_bf16(c < l ? v : 0.0f, hi, lo);
        xt[(int64_t)c * rows + r] = hi;
        xt[((int64_t)lp + c) * rows + r] = lo;
      }
    }
  }
}

// ============================================================== projection
// btp[s] = (A[rows of chunk s, :])^T Q[rows of chunk s, :]   (n x l, fp32)
// with Q given transposed as bf16 hi + lo (2 x lp x m). WG: 128 columns of A,
// 4 waves x 32 columns. Per step, 64 rows of A (bf16 or fp32) and the
// matching 64 columns of Q^T (hi, lo) pass through LDS; the next step's
// pieces are loaded into registers while the current step is multiplied.
template <typename T, int NC = 0>
__global__ void __launch_bounds__(kThreads) project_kernel(const T *__restrict__ A, int64_t m, int64_t n, int64_t lda,
                                                           const unsigned short *__restrict__ qt, int l, int lp,
                                                           int64_t chunk_rows, float *__restrict__ btp) {
  // blockIdx.z selects a tile of kLpMax columns of Q starting at l0
  const int l0 = blockIdx.z * kLpMax;
  const int lt = min(kLpMax, lp - l0);
  constexpr int KS = 64;
  constexpr int TN = 128;
  constexpr int NT = (sizeof(T) == 4) ? 3 : 1;
  constexpr int PIECE = 16 / sizeof(T);                      // elements per 16-byte piece
  constexpr int APR = KS * (TN / PIECE) / kThreads;          // A pieces per thread per step
  constexpr int QPR = (2 * kLpMax * (KS / 8) + kThreads - 1) / kThreads;  // Q^T pieces
  __shared__ __attribute__((aligned(16))) T at[KS][TN + (sizeof(T) == 2 ? 8 : 4)];
  __shared__ __attribute__((aligned(16))) unsigned short qs[2][kLpMax][KS + 8];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t col0 = (int64_t)blockIdx.x * TN;
  const int s = blockIdx.y;
  const int64_t r_beg = (int64_t)s * chunk_rows;
  const int64_t r_end = std::min<int64_t>(m, r_beg + chunk_rows);
  // NC > 0: exactly NC 16-column tiles of Q (as in the sketch)
  constexpr int NCM = NC ? NC : kLpMax / 16;
  const int nit = NC ? NC : lt >> 4;
  floatx4 acc[2][NCM];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NCM; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[APR], rq[QPR];
  auto load = [&](int64_t r0) {
#pragma unroll
    for (int p = 0; p < APR; ++p) {
      const int idx = t + kThreads * p;
      const int rr = idx / (TN / PIECE), q = idx % (TN / PIECE);
      const int64_t row = r0 + rr, col = col0 + q * PIECE;
      ra[p] = (row < r_end && col < n) ? *(const uint4 *)(A + row * lda + col) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int p = 0; p < QPR; ++p) {
      const int idx = t + kThreads * p;
      const int h = idx / (lt * (KS / 8)), rem = idx % (lt * (KS / 8));
      const int i = rem / (KS / 8), q = rem % (KS / 8);
      const int64_t row = r0 + q * 8;
      rq[p] = (idx < 2 * lt * (KS / 8) && row < r_end)
                  ? *(const uint4 *)(qt + ((int64_t)h * lp + l0 + i) * m + row)
                  : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int p = 0; p < APR; ++p) {
      const int idx = t + kThreads * p;
      *(uint4 *)&at[idx / (TN / PIECE)][(idx % (TN / PIECE)) * PIECE] = ra[p];
    }
#pragma unroll
    for (int p = 0; p < QPR; ++p) {
      const int idx = t + kThreads * p;
      if (idx < 2 * lt * (KS / 8)) {
        const int h = idx / (lt * (KS / 8)), rem = idx % (lt * (KS / 8));
        *(uint4 *)&qs[h][rem / (KS / 8)][(rem % (KS / 8)) * 8] = rq[p];
      }
    }
  };

  if (r_beg < r_end) load(r_beg);
  for (int64_t r0 = r_beg; r0 < r_end; r0 += KS) {
    __syncthreads();
    store();
    if (r0 + KS < r_end) load(r0 + KS);  // in flight while this step is multiplied
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < KS / 32; ++kq) {
      // both column sets' A fragments first, so each Q^T fragment read from
      // LDS feeds the MFMAs of both
      ushortx8 af[2][NT];
#pragma unroll
      for (int cs = 0; cs < 2; ++cs) {
        const int cl = wave * 32 + cs * 16 + r16;  // A column inside the tile
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (sizeof(T) == 2) {
            af[cs][0][e] = at[kq * 32 + g * 8 + e][cl];
          } else {
            const float x = at[kq * 32 + g * 8 + e][cl];
            const unsigned short hi = f32_to_bf16(x);
            const float r1 = x - bf16_to_f32(hi);
            const unsigned short mid = f32_to_bf16(r1);
            af[cs][0][e] = hi;
            af[cs][NT > 1 ? 1 : 0][e] = mid;
            af[cs][NT > 2 ? 2 : 0][e] = f32_to_bf16(r1 - bf16_to_f32(mid));
          }
        }
      }
#pragma unroll
      for (int it = 0; it < NCM; ++it) {
        if (NC || it < nit) {
          const ushortx8 qh = *(const ushortx8 *)&qs[0][it * 16 + r16][kq * 32 + g * 8];
          const ushortx8 ql = *(const ushortx8 *)&qs[1][it * 16 + r16][kq * 32 + g * 8];
#pragma unroll
          for (int cs = 0; cs < 2; ++cs)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
              acc[cs][it] = mfma16_bf16(af[cs][tt], qh, acc[cs][it]);
              acc[cs][it] = mfma16_bf16(af[cs][tt], ql, acc[cs][it]);
            }
        }
      }
    }
  }
  float *out = btp + (int64_t)s * n * l;
#pragma unroll
  for (int cs = 0; cs < 2; ++cs)
#pragma unroll
    for (int it = 0; it < NCM; ++it) {
      if (NC || it < nit) {
        const int i = l0 + it * 16 + r16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = col0 + wave * 32 + cs * 16 + g * 4 + q;
          if (col < n && i < l) out[col * l + i] = acc[cs][it][q];
        }
      }
    }
}

// ================================================ tridiagonal reduction
// Householder reduction of the symmetric l x l matrix G (upper triangle read,
// fp64) to tridiagonal T = H^T G H, H = H_0 ... H_{l-3}, in one workgroup of
// four waves with one barrier per reflector. Lane c holds columns c and
// c + 64 of the rows r = wave + 4 i (both triangles) in registers. Step j,
// with x = row j right of its diagonal (the reflector maps it to
// alpha e_{j+1}: v = x - alpha e_{j+1}, beta = 2 / v.v):
//  - by symmetry each wave's rows give a partial of A x over all columns
//    (sum_r A[r][c] x_r, the x_r of its rows through a wave-private LDS
//    list); the partials meet in LDS across the barrier, with a copy of row
//    j + 1 left by its owner. Since A v = A x - alpha A[j + 1], |x|, alpha
//    and beta (square root, reciprocal) are formed by every wave alongside
//    the products instead of ahead of them;
//  - after the barrier every wave sums the partials in one order, so all
//    hold the same p = beta A v, K = beta p.v / 2 and w = p - K v; it
//    forms row j + 1 after the update (T's diagonal entry and the next x)
//    and applies A -= v w^T + w v^T to its rows. Rows at or above j are left
//    as they are (v and p vanish there), and row j + 1 is never read again,
//    so every row takes the update with v_r = x_r, branch free.
// Columns at or left of j keep their values (p and v vanish there).
// T (diagonal, off-diagonal), the beta_j and the reflectors go to global
// memory for the eigenpair kernels.
constexpr int kTriThreads = 256;

// x at position idx (uniform) of a lane-distributed vector (column c in lane
// c % 64, slot c / 64)
template <int NS>
__device__ __forceinline__ double lane_value(const double (&x)[NS], int idx) {
  if (NS == 1 || idx < 64) return readlane_f64(x[0], idx & 63);
  return readlane_f64(x[NS - 1], idx & 63);
}

// RPW: rows per wave (r = wave + 4 i), 4 RPW >= l; lp = 80 takes 20.
template <int NS, int RPW = NS == 1 ? 16 : kLpMax / 4>
__global__ void __launch_bounds__(kTriThreads)
    tridiag_kernel(const double *__restrict__ g, int l, int lp, double *__restrict__ dg_out,
                   double *__restrict__ eo_out, double *__restrict__ beta_out, double *__restrict__ v_out) {
  static_assert(kLpMax <= 128 && kLpMax % 16 == 0, "two column slots, rows below 128");
  static_assert(RPW % 2 == 0 && 4 * RPW <= 64 * NS, "rows read in pairs, within the column slots");
  __shared__ double qp[2][4][64 * NS];
  __shared__ double yb[2][64 * NS];
  // per wave: x and p at its own rows (entry i: row wave + 4 i; entries
  // RPW + lane take the writes of lanes holding other rows), written and
  // read by that wave alone
  __shared__ __attribute__((aligned(16))) double xl[4][RPW + 64], pl[4][RPW + 64];
  __shared__ double td[kLpMax + 64], te[kLpMax + 64], tb[kLpMax + 64];  // T and beta (+ discard slots)
  const int n = l, t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  double a[RPW][NS];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = w + 4 * i;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = lane + 64 * s;
      const int lo = r < c ? r : c, hi = r < c ? c : r;
      a[i][s] = (r < n && c < n) ? g[lo * lp + hi] : 0.0;
    }
  }
  for (int i = t; i < kLpMax; i += kTriThreads) {
    td[i] = 0.0;
    te[i] = 0.0;
    tb[i] = 0.0;
  }
  for (int e = t; e < lp * lp; e += kTriThreads)
    if (e >= (n > 2 ? n - 2 : 0) * lp) v_out[e] = 0.0;
  // the wave's entries of a lane-distributed vector, by its own rows (every
  // lane writes: those of other rows into the discard slot)
  auto own_rows = [&](const double (&x)[NS], double *lst) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = lane + 64 * s;
      lst[((c & 3) == w && (c >> 2) < RPW) ? (c >> 2) : RPW + lane] = x[s];
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto read_rows = [&](const double *lst, double (&out)[RPW]) {
#pragma unroll
    for (int i = 0; i < RPW; i += 2) {
      const double2 d2 = *(const double2 *)&lst[i];
      out[i] = d2.x;
      out[i + 1] = d2.y;
    }
  };
  double xv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int c = lane + 64 * s;
    xv[s] = (c > 0 && c < n) ? g[c] : 0.0;
  }
  __syncthreads();
  if (t == 0) td[0] = n > 0 ? g[0] : 0.0;
  // |x|, alpha and beta of the reflector for x (row j right of its
  // diagonal). Each step forms the next step's values as soon as the next x
  // is known, so their reduction, square root and reciprocal run between
  // the update's multiply-adds instead of ahead of the next matrix-vector
  // product.
  double nrm2, alpha, beta;
  auto reflector = [&](int j) {
    double x2 = 0.0;
#pragma unroll
    for (int s = 0; s < NS; ++s) x2 = fma(xv[s], xv[s], x2);
    nrm2 = wave_sum_f64(x2);
    const double x0 = lane_value(xv, j + 1), nrm = sqrt(nrm2);
    alpha = x0 >= 0.0 ? -nrm : nrm;
    beta = nrm2 > 0.0 ? recip_f64(nrm * (nrm + fabs(x0))) : 0.0;
  };
  reflector(0);

  for (int j = 0; j + 2 < n; ++j) {
    const int buf = j & 1;
    // ---- this wave's partial of A x
    double xr[RPW];
    own_rows(xv, xl[w]);
    read_rows(xl[w], xr);
    double q4[4][NS];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s) q4[u][s] = 0.0;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int s = 0; s < NS; ++s) q4[i & 3][s] = fma(a[i][s], xr[i], q4[i & 3][s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) qp[buf][w][lane + 64 * s] = (q4[0][s] + q4[1][s]) + (q4[2][s] + q4[3][s]);
    if (w == ((j + 1) & 3)) {
#pragma unroll
      for (int i = 0; i < RPW; ++i)
        if (w + 4 * i == j + 1) {
#pragma unroll
          for (int s = 0; s < NS; ++s) yb[buf][lane + 64 * s] = a[i][s];
        }
    }
    __syncthreads();
    // ---- v, p = beta (A x - alpha A[j + 1]), K, w
    double v[NS], pv[NS], wv[NS], pvs = 0.0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = lane + 64 * s;
      v[s] = c == j + 1 ? xv[s] - alpha : xv[s];
      const double sum = ((qp[buf][0][c] + qp[buf][1][c]) + qp[buf][2][c]) + qp[buf][3][c];
      pv[s] = (c > j && c < n) ? beta * fma(-alpha, yb[buf][c], sum) : 0.0;
      pvs = fma(pv[s], v[s], pvs);
    }
    double pr[RPW];
    own_rows(pv, pl[w]);
    read_rows(pl[w], pr);
    const double K = 0.5 * beta * wave_sum_f64(pvs);
#pragma unroll
    for (int s = 0; s < NS; ++s) wv[s] = fma(-K, v[s], pv[s]);
    // ---- row j + 1 after the update: T's diagonal entry and the next x
    const double v1 = lane_value(v, j + 1), w1 = lane_value(wv, j + 1);
    double dnext = 0.0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = lane + 64 * s;
      const double xn = fma(-v1, wv[s], fma(-w1, v[s], yb[buf][c]));
      dnext = c == j + 1 ? xn : dnext;
      xv[s] = (c > j + 1 && c < n) ? xn : 0.0;
    }
    const double alpha_j = alpha, beta_j = beta;
    reflector(j + 1);
    // ---- A -= v w^T + w v^T on every row
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const double wr = fma(-K, xr[i], pr[i]);
#pragma unroll
      for (int s = 0; s < NS; ++s) a[i][s] = fma(-xr[i], wv[s], fma(-wr, v[s], a[i][s]));
    }
    // ---- outputs of the step: T's entries (LDS, written out at the end)
    // and the reflector
    if (w == 0) {
      td[lane == ((j + 1) & 63) ? j + 1 : kLpMax + lane] = dnext;
      te[lane == 0 ? j : kLpMax + lane] = alpha_j;
      tb[lane == 0 ? j : kLpMax + lane] = beta_j;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (lane + 64 * s < lp) v_out[(int64_t)j * lp + lane + 64 * s] = v[s];
    }
  }
  // the last off-diagonal (no reflector) and the last diagonal entry
  if (n >= 2) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (w == 0 && lane + 64 * s == n - 1) te[n - 2] = xv[s];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if (w + 4 * i == n - 1) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (lane + 64 * s == n - 1) td[n - 1] = a[i][s];
      }
  }
  __syncthreads();
  for (int i = t; i < lp; i += kTriThreads) {
    dg_out[i] = i < n ? td[i] : 0.0;
    eo_out[i] = i + 1 < n ? te[i] : 0.0;
    beta_out[i] = i + 2 < n ? tb[i] : 0.0;
  }
}

// ================================================================ assemble
// U[r][c] = sum_t Q[r][t] E[t][c] (fp64 accumulate) over the workgroup's
// chunk of rows, and the chunk's argmax of |U[:, c]| (lowest row on ties)
// with its signed value. Thread (rg, c) owns 16 consecutive rows of column c:
// one E load feeds 16 FMAs against broadcast reads of the staged Q rows.

__global__ void __launch_bounds__(kThreads)
    assemble_u_kernel(const float *__restrict__ q, int64_t m, int l, int lp, int k, const double *__restrict__ evec,
                      int64_t chunk_rows, float *__restrict__ U, float *__restrict__ am_val, int *__restrict__ am_idx) {
  __shared__ double E[kLpMax][kLpMax];
  __shared__ float qs[kAsmRows * kAsmGroups][kLpMax + 1];
  __shared__ float bv[kThreads], bsv[kThreads];
  __shared__ int bix[kThreads];
  const int t = threadIdx.x;
  const int groups = asm_groups(k);
  const int c = t % k, rg = t / k;
  const bool active = rg < groups;
  const int64_t r0 = blockIdx.x * chunk_rows;
  const int nrows = (int)std::min<int64_t>(chunk_rows, m - r0);
  stage_batched<16>(&E[0][0], evec, l * k, [=](int i) { return (i / k) * lp + i % k; },
                    [=](int i) { return (i / k) * kLpMax + i % k; });
  stage_batched<16>(&qs[0][0], q + r0 * l, nrows * l, [](int i) { return i; },
                    [=](int i) { return (i / l) * (kLpMax + 1) + i % l; });
  __syncthreads();
  float best_abs = -1.0f, best_val = 0.0f;
  int best_idx = 0x7FFFFFFF;
  if (active) {
    double acc[kAsmRows];
#pragma unroll
    for (int r = 0; r < kAsmRows; ++r) acc[r] = 0.0;
    const int rbase = rg * kAsmRows;
    for (int q2 = 0; q2 < l; ++q2) {
      const double e = E[q2][c];
#pragma unroll
      for (int r = 0; r < kAsmRows; ++r) acc[r] += (double)qs[rbase + r][q2] * e;
    }
#pragma unroll
    for (int r = 0; r < kAsmRows; ++r) {
      const int rr = rbase + r;
      if (rr < nrows) {
        const float u = (float)acc[r];
        U[(r0 + rr) * k + c] = u;
        if (fabsf(u) > best_abs) {
          best_abs = fabsf(u);
          best_val = u;
          best_idx = (int)(r0 + rr);
        }
      }
    }
  }
  bv[t] = active ? best_abs : -1.0f;
  bsv[t] = active ? best_val : 0.0f;
  bix[t] = active ? best_idx : 0x7FFFFFFF;
  __syncthreads();
  if (t < k) {
    float ba = -1.0f, bval = 0.0f;
    int bi = 0x7FFFFFFF;
    for (int g = 0; g < groups; ++g) {
      const int w = g * k + t;
      if (bv[w] > ba || (bv[w] == ba && bix[w] < bi)) {
        ba = bv[w];
        bval = bsv[w];
        bi = bix[w];
      }
    }
    am_val[blockIdx.x * k + t] = bval;
    am_idx[blockIdx.x * k + t] = bi;
  }
}

// V[j][c] = (sum_t B^T[j][t] E[t][c]) / sigma_c   (0 for dropped sigma), with
// the same 16-rows-per-thread blocking (the fp64 sum is scaled once).
__global__ void __launch_bounds__(kThreads)
    assemble_v_kernel(const float *__restrict__ bt, int64_t n, int l, int lp, int k, const double *__restrict__ evec,
                      const double *__restrict__ sig_inv, float *__restrict__ V) {
  __shared__ double E[kLpMax][kLpMax];
  __shared__ float bs[kAsmRows * kAsmGroups][kLpMax + 1];
  const int t = threadIdx.x;
  const int groups = asm_groups(k);
  const int c = t % k, rg = t / k;
  const int64_t chunk_rows = asm_chunk_rows(k);
  const int64_t r0 = blockIdx.x * chunk_rows;
  const int nrows = (int)std::min<int64_t>(chunk_rows, n - r0);
  const double sc = rg < groups ? sig_inv[c] : 0.0;
  stage_batched<16>(&E[0][0], evec, l * k, [=](int i) { return (i / k) * lp + i % k; },
                    [=](int i) { return (i / k) * kLpMax + i % k; });
  stage_batched<16>(&bs[0][0], bt + r0 * l, nrows * l, [](int i) { return i; },
                    [=](int i) { return (i / l) * (kLpMax + 1) + i % l; });
  __syncthreads();
  if (rg >= groups) return;
  double acc[kAsmRows];
#pragma unroll
  for (int r = 0; r < kAsmRows; ++r) acc[r] = 0.0;
  const int rbase = rg * kAsmRows;
  for (int q2 = 0; q2 < l; ++q2) {
    const double e = E[q2][c];
#pragma unroll
    for (int r = 0; r < kAsmRows; ++r) acc[r] += (double)bs[rbase + r][q2] * e;
  }
#pragma unroll
  for (int r = 0; r < kAsmRows; ++r)
    if (rbase + r < nrows) V[(r0 + rbase + r) * k + c] = (float)(acc[r] * sc);
}

// sign[c] = -1 if the largest-|U[:, c]| entry (lowest row on ties) is negative
// Column c's sign from the chunk argmax partials: the largest |U[:, c]|,
// lowest row on ties (an order-independent selection). Eight groups of 128
// threads scan every eighth partial, then group 0 combines the eight.
__global__ void __launch_bounds__(1024)
    sign_kernel(const float *__restrict__ am_val, const int *__restrict__ am_idx, int parts, int k,
                float *__restrict__ sign) {
  __shared__ float pa[8][128], pv[8][128];
  __shared__ int pi[8][128];
  const int c = threadIdx.x & 127, g = threadIdx.x >> 7;
  float ba = -1.0f, bv = 0.0f;
  int bi = 0x7FFFFFFF;
  if (c < k) {
    // sixteen partials per batch, their loads in flight together
    constexpr int PER = 16;
    for (int p0 = g; p0 < parts; p0 += 8 * PER) {
      float vv[PER];
      int ii[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int p = p0 + 8 * u;
        vv[u] = p < parts ? am_val[p * k + c] : 0.0f;
        ii[u] = p < parts ? am_idx[p * k + c] : 0x7FFFFFFF;
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const float v = vv[u];
        const int i = ii[u];
        if (p0 + 8 * u < parts && (fabsf(v) > ba || (fabsf(v) == ba && i < bi))) {
          ba = fabsf(v);
          bv = v;
          bi = i;
        }
      }
    }
  }
  pa[g][c] = ba;
  pv[g][c] = bv;
  pi[g][c] = bi;
  __syncthreads();
  if (g == 0 && c < k) {
    for (int q = 1; q < 8; ++q)
      if (pa[q][c] > ba || (pa[q][c] == ba && pi[q][c] < bi)) {
        ba = pa[q][c];
        bv = pv[q][c];
        bi = pi[q][c];
      }
    sign[c] = bv < 0.0f ? -1.0f : 1.0f;
  }
}

// max |x| over a rows x cols fp32 matrix (row stride ld) into *out (bits).
__global__ void amax_f32_kernel(const float *__restrict__ x, int64_t rows, int64_t cols, uint32_t *out) {
  float mx = 0.0f;
  const int64_t total = rows * cols;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x)
    mx = fmaxf(mx, fabsf(x[i]));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(mx));
}

// ================================================================= factors
// For X = U (m x k, y = 0) or V (n x k, y = 1): flip column signs in place,
// quantize X^T along its length into (codes, scales), and write the bf16
// hi/lo panel of X * mult (mult = 1 for U, S for V) for the residual MFMA.
// Thread = (column c < kp, block of B rows).
template <bool NV>
__global__ void __launch_bounds__(kThreads)
    factor_kernel(float *__restrict__ U, float *__restrict__ V, int64_t m, int64_t n, int k, int kp,
                  const float *__restrict__ sign, const float *__restrict__ S, uint8_t *__restrict__ ucodes,
                  uint8_t *__restrict__ uscales, float *__restrict__ uts, uint8_t *__restrict__ vcodes,
                  uint8_t *__restrict__ vscales, float *__restrict__ vts, const uint32_t *__restrict__ amax,
                  unsigned short *__restrict__ uhl, unsigned short *__restrict__ whl) {
  constexpr int B = NV ? 16 : 32;
  const bool isv = blockIdx.y == 1;
  float *X = isv ? V : U;
  const int64_t rows = isv ? n : m;
  uint8_t *codes = isv ? vcodes : ucodes;
  uint8_t *scales = isv ? vscales : uscales;
  unsigned short *hl = isv ? whl : uhl;
  const int64_t idx = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  const int c = (int)(idx % kp);
  const int64_t blk = idx / kp;
  if (blk >= rows / B) return;
  float s_t = 1.0f;
  if (NV) {
    s_t = nv_tensor_scale(__uint_as_float(amax[isv ? 1 : 0]));
    if (idx == 0) *(isv ? vts : uts) = s_t;
  }
  if (c >= k) {
    for (int i = 0; i < B; ++i) {
      hl[(blk * B + i) * kp + c] = 0;
      hl[rows * kp + (blk * B + i) * kp + c] = 0;
    }
    return;
  }
  const float sg = sign[c];
  const float mult = isv ? S[c] : 1.0f;
  float v[B];
#pragma unroll
  for (int i = 0; i < B; ++i) v[i] = X[(blk * B + i) * k + c];  // all loads before the first store
#pragma unroll
  for (int i = 0; i < B; ++i) {
    v[i] *= sg;
    X[(blk * B + i) * k + c] = v[i];
    unsigned short h, w;
    split_bf16(v[i] * mult, h, w);
    hl[(blk * B + i) * kp + c] = h;
    hl[rows * kp + (blk * B + i) * kp + c] = w;
  }
  float amx = 0.0f;
  for (int i = 0; i < B; ++i) amx = fmaxf(amx, fabsf(v[i]));
  uint32_t sb;
  uint32_t pk[B / 8];
  if (!NV) {
    const int se = mx_shared_exponent(amx);
    sb = (uint32_t)(se + 127);
    e2m1_pack_scaled<B>(v, pow2_f32(se), pk);
  } else {
    sb = e4m3_rne_sat(__fdiv_rn(amx, 6.0f * s_t));
    const float den = e4m3_value(sb) * s_t;
    float q[B];
    for (int i = 0; i < B; ++i) q[i] = sb ? __fdiv_rn(v[i], den) : v[i] * 0.0f;  // zero scale: signs only
    e2m1_pack<B>(q, pk);
  }
  uint32_t *dst = (uint32_t *)(codes + (int64_t)c * (rows / 2) + blk * (B / 2));
  for (int w = 0; w < B / 8; ++w) dst[w] = pk[w];
  scales[(int64_t)c * (rows / B) + blk] = (uint8_t)sb;
}

// ================================================================ residual
// R = A - U diag(S) V^T on a 128 x 128 tile, then block quantization of R
// along n (R_q) and along m (Rt_q) from the same LDS copy. L = U W^T with
// W = V S comes from bf16 MFMA on hi/lo panels: Uh Wh + Uh Wl + Ul Wh.
// AMAX_ONLY: only the tensor max of |R| (NVFP4 tensor scale) is produced.
constexpr int kRT = 128;  // residual tile rows
constexpr int kRC = 64;   // residual tile columns (a 34 KB LDS tile: four workgroups per CU)

template <int B, bool NV>
__device__ __forceinline__ void quant_store(const float (&v)[B], float s_t, uint8_t *codes, uint8_t *scale) {
  float amx = 0.0f;
#pragma unroll
  for (int i = 0; i < B; ++i) amx = fmaxf(amx, fabsf(v[i]));
  uint32_t sb;
  uint32_t pk[B / 8];
  if (!NV) {
    const int se = mx_shared_exponent(amx);
    sb = (uint32_t)(se + 127);
    e2m1_pack_scaled<B>(v, pow2_f32(se), pk);
  } else {
    sb = e4m3_rne_sat(__fdiv_rn(amx, 6.0f * s_t));
    const float den = e4m3_value(sb) * s_t;
    float q[B];
#pragma unroll
    for (int i = 0; i < B; ++i) q[i] = sb ? __fdiv_rn(v[i], den) : v[i] * 0.0f;  // zero scale: signs only
    e2m1_pack<B>(q, pk);
  }
  if constexpr (B == 32) {
    *(uint4 *)codes = uint4{pk[0], pk[1], pk[2], pk[3]};
  } else {
    *(uint2 *)codes = uint2{pk[0], pk[1]};
  }
  *scale = (uint8_t)sb;
}

// Barrier for LDS traffic only: this wave's LDS accesses are complete, its
// global loads and stores may still be in flight (the loads of the next tile
// must stay in flight across the tile's barriers).
#define METIS_LDS_BARRIER()                                                       \
  do {                                                                            \
    __asm__ volatile("" ::: "memory");                                           \
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));                        \
    __builtin_amdgcn_s_barrier();                                                 \
    __asm__ volatile("" ::: "memory");                                           \
  } while (0)

// XCDs of the chip; workgroups go to them round robin by block index.
constexpr int kXcds = 8;

// Residual + quantization over kRT x kRC tiles, persistent. The tiles are
// taken in blocks of 2 x 4 (256 rows x 256 columns: whole 128-byte lines of
// the rows of R (32 code bytes per tile row) and of R^T (64 per tile
// column)), each block by a group of eight workgroups on one XCD, one tile
// each (member j: row tile 2 s + j / 4, column tile 4 c + j % 4 of block
// (s, c)), so the pieces of a line are written together and meet in one L2
// before it writes the line back. A group walks a run of w blocks along the
// rows; XCD x takes the groups of a contiguous stretch of runs (block index
// b goes to XCD b % 8). Tiles past the matrix edge store nothing. Per tile: L by
// MFMA (U of the tile's rows in registers, reloaded when the row tile
// changes; the W panel of the tile's columns staged in LDS), R = A - L kept
// in the LDS tile, row blocks quantized along n, then column blocks along m.
// The W panel and A blocks of the next tile load during the current one.
// Global loads take clamped, always valid addresses (m and n are multiples of
// 32), so no branch separates a load from its use and the waits stay counted.
// MEAN: the mean-residual split, L[r][c] = mu[c] (fp32, passed as `mu`)
// instead of the MFMA product, so R = A - mu is one fp32 subtraction.
constexpr int kResGroup = 8;  // workgroups per block of 2 x 4 tiles
// KP: the factor rank padded to 32 (32, 64 or 96), fixed at compile time so
// every panel load and MFMA step is used and the loop bounds are static.
template <typename T, bool NV, bool AMAX_ONLY, bool MEAN, int KP>
__global__ void __launch_bounds__(kThreads, 2)  // two waves per SIMD: 256 registers
    residual_kernel(const T *__restrict__ A, int64_t m, int64_t n, int64_t lda, const unsigned short *__restrict__ uhl,
                    const unsigned short *__restrict__ whl, uint8_t *__restrict__ rcodes,
                    uint8_t *__restrict__ rscales, float *__restrict__ rts, uint8_t *__restrict__ tcodes,
                    uint8_t *__restrict__ tscales, float *__restrict__ tts, uint32_t *__restrict__ amax,
                    const float *__restrict__ mu = nullptr) {
  constexpr int B = NV ? 16 : 32;
  __shared__ __attribute__((aligned(16))) float lt[kRT][kRC + 4];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, g = lane >> 4;
  // ---- this workgroup's run of blocks (the grid is 8 x 8 x groups per XCD)
  const int ctiles = (int)cdiv(n, kRC), rtiles = (int)cdiv(m, kRT);
  const int cblocks = (ctiles + 3) / 4, nblk = (rtiles + 1) / 2 * cblocks;
  const int ngrp = (int)gridDim.x / kResGroup, gpx = ngrp / kXcds;
  const int bx = (int)blockIdx.x, kx = bx / kXcds;
  const int grp = (bx % kXcds) * gpx + kx / kResGroup, member = kx % kResGroup;
  const int parity = member / 4, cofs = member % 4;
  const int w = (nblk + ngrp - 1) / ngrp;
  const int p0 = grp * w, p1 = min(nblk, p0 + w);
  if (p0 >= p1) return;
  // A row block b = t + 256 j of a tile is row b / RPB, columns (b % RPB) * B ..
  constexpr int RPB = kRC / B;                 // blocks per tile row
  constexpr int NJ = kRT * RPB / kThreads;     // row blocks per thread
  constexpr int VEC = B * (int)sizeof(T) / 16;  // 16-byte pieces per block
  static_assert(NJ * kThreads == kRT * RPB, "row blocks must divide over the threads");
  static_assert(KP == 32 || KP == 64 || KP == 96, "factor rank padded to 32, at most 96");
  constexpr int kp = KP;
  // 16-byte pieces of the W panel (hi, lo) per thread; none in the mean split
  constexpr int PW = MEAN ? 0 : 2 * kRC * (kp / 8) / kThreads;
  static_assert(MEAN || PW * kThreads == 2 * kRC * (kp / 8), "the W panel divides over the threads");
  // what a tile needs from HBM apart from U: its A blocks and its W panel
  struct Pre {
    uint4 a[NJ][VEC];
    uint4 w[PW > 0 ? PW : 1];
  };
  auto tile_rt = [&](int p) { return 2 * (p / cblocks) + parity; };
  auto tile_ct = [&](int p) { return 4 * (p % cblocks) + cofs; };
  // Loads of this workgroup's tile of block p into pre: the panel first, then
  // A. Rows or columns past the matrix (a skipped tile's too) are loaded
  // clamped, never stored.
  auto load_pre = [&](int p, Pre &pre) {
    const int64_t row0 = (int64_t)tile_rt(p) * kRT, col0 = (int64_t)tile_ct(p) * kRC;
    if constexpr (!MEAN) {
      const int64_t wn = n * kp;
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const int idx = t + u * kThreads;
        const int h = idx / (kRC * (kp / 8)), rem = idx % (kRC * (kp / 8));
        const int c = rem / (kp / 8), qq = rem % (kp / 8);
        pre.w[u] = *(const uint4 *)(whl + h * wn + min(col0 + c, n - 1) * kp + qq * 8);
      }
      // panel, then A, everywhere (the first tile's loads too): the waits at
      // the loop head assume one order
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      const int b = t + kThreads * jb, rr = b / RPB, cb = b % RPB;
      const int64_t row = min(row0 + rr, m - 1), col = min(col0 + cb * B, n - B);
      const uint4 *src = (const uint4 *)(A + row * lda + col);
#pragma unroll
      for (int qq = 0; qq < VEC; ++qq) pre.a[jb][qq] = src[qq];
    }
  };
  float s_t = 1.0f;
  if (NV && !AMAX_ONLY) s_t = nv_tensor_scale(__uint_as_float(*amax));
  if (NV && !AMAX_ONLY && bx == 0 && t == 0) {
    if (rts) *rts = s_t;
    if (tts) *tts = s_t;
  }
  ushortx8 uh[kp / 32][2], ul[kp / 32][2];
  int cur_rt = -1;
  float mx = 0.0f;
  // One tile: `cur` holds its loads (issued one tile earlier), `nxt`
  // receives the next tile's (the last tile of the run loads itself again,
  // from cache), so the waits of a tile are for loads a tile old.
  auto tile = [&](int p, Pre &cur, Pre &nxt) {
    const int rt = tile_rt(p), ct = tile_ct(p);
    const int64_t row0 = (int64_t)rt * kRT, col0 = (int64_t)ct * kRC;
    // a tile past the matrix edge runs like the others on clamped loads; the
    // row and column checks below keep all of its stores out (a branch
    // around it would cost the loop its counted waits)
    const int p_n = min(p + 1, p1 - 1);
    if constexpr (MEAN) {
      // each thread fills a quarter of a column of the tile with mu
      constexpr int RF = kRT * kRC / kThreads;
      const int c = t % kRC, r0 = (t / kRC) * RF;
      const float v = mu[min(col0 + c, n - 1)];
      load_pre(p_n, nxt);
#pragma unroll 8
      for (int r = 0; r < RF; ++r) lt[r0 + r][c] = v;
    } else {
      // ---- L tile via MFMA: wave owns rows wave*32 .. +32, all kRC columns.
      // The W panel (hi, lo) of the tile's columns is shared by the four
      // waves and staged in LDS, in the space the R tile takes later (row
      // stride kp + 8 bf16 keeps the fragment reads conflict free).
      unsigned short *wst = (unsigned short *)&lt[0][0];  // [2][kRC][kp + 8]
      static_assert(2 * kRC * (kp + 8) * 2 <= kRT * (kRC + 4) * 4, "the W panel fits the tile's LDS");
      const int wstride = kp + 8;
      const int64_t um = m * kp;
      if (rt != cur_rt) {
        cur_rt = rt;
#pragma unroll
        for (int ks = 0; ks < kp / 32; ++ks)
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            // rows past m are loaded clamped: their products land in rows of
            // L that are never stored
            const int64_t row = min(row0 + wave * 32 + rs * 16 + r16, m - 1);
            const unsigned short *pu = uhl + row * kp + ks * 32 + g * 8;
            uh[ks][rs] = *(const ushortx8 *)pu;
            ul[ks][rs] = *(const ushortx8 *)(pu + um);
          }
        // wait for U here, in the (rare) reload: the loads were issued after
        // the previous tile's stores, so waiting for them later would make
        // every tile wait for those stores
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
      }
      load_pre(p_n, nxt);
      // every load of the next tile is issued before this tile's data is
      // waited for, so those waits never reach back to the previous stores
      __builtin_amdgcn_sched_barrier(0);
      // piece idx of the panel goes to LDS row idx / P, slot idx % P
      // (P = kp / 8)
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const int idx = t + u * kThreads;
        *(uint4 *)(wst + (idx / (kp / 8)) * wstride + (idx % (kp / 8)) * 8) = cur.w[u];
      }
      METIS_LDS_BARRIER();
      constexpr int NCS = kRC / 16;
      floatx4 acc[2][NCS];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NCS; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kp / 32; ++ks) {
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
          const int c = cs * 16 + r16;
          const ushortx8 wh = *(const ushortx8 *)(wst + c * wstride + ks * 32 + g * 8);
          const ushortx8 wl = *(const ushortx8 *)(wst + (kRC + c) * wstride + ks * 32 + g * 8);
#pragma unroll
          for (int rs = 0; rs < 2; ++rs) {
            acc[rs][cs] = mfma16_bf16(uh[ks][rs], wh, acc[rs][cs]);
            acc[rs][cs] = mfma16_bf16(uh[ks][rs], wl, acc[rs][cs]);
            acc[rs][cs] = mfma16_bf16(ul[ks][rs], wh, acc[rs][cs]);
          }
        }
      }
      METIS_LDS_BARRIER();  // the W panel is no longer read
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) lt[wave * 32 + rs * 16 + g * 4 + qq][cs * 16 + r16] = acc[rs][cs][qq];
    }
    METIS_LDS_BARRIER();
    // the A registers pass through an empty asm here, so their conversion
    // to fp32 is not hoisted into the tile that issued the loads (where it
    // would wait for them)
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
      for (int qq = 0; qq < VEC; ++qq)
        __asm__ volatile("" : "+v"(cur.a[jb][qq].x), "+v"(cur.a[jb][qq].y), "+v"(cur.a[jb][qq].z),
                         "+v"(cur.a[jb][qq].w));
    // ---- row blocks (along n): R = A - L, kept in LDS for the column pass
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      const int b = t + kThreads * jb, rr = b / RPB, cb = b % RPB;
      const int64_t row = row0 + rr, col = col0 + cb * B;
      float v[B];
      const bool ok = row < m && col < n;
      const T *pa = (const T *)&cur.a[jb][0];
      // computed for every block (a block past the edge holds clamped A and
      // never reaches an in-range block of either orientation, as m and n are
      // multiples of B); `ok` only masks the tensor max and the stores, so no
      // branch holds a use of the loaded registers and their waits stay counted
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = load_f32(pa + i) - lt[rr][cb * B + i];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        lt[rr][cb * B + i] = v[i];
        mx = fmaxf(mx, ok ? fabsf(v[i]) : 0.0f);
      }
      if (!AMAX_ONLY && ok && rcodes)
        quant_store<B, NV>(v, s_t, rcodes + row * (n / 2) + col / 2, rscales + row * (n / B) + col / B);
    }
    if (!AMAX_ONLY && tcodes) {
      METIS_LDS_BARRIER();
      // ---- column blocks (along m) into R^T (n x m): thread t takes
      // consecutive row blocks of column t % kRC, so its code stores are
      // adjacent in R^T's row
      constexpr int PER = kRC * (kRT / B) / kThreads;  // row blocks per thread
      const int cc = t % kRC, rb0 = (t / kRC) * PER;
      const int64_t col = col0 + cc;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int rb = rb0 + u;
        const int64_t row = row0 + rb * B;
        if (col >= n || row >= m) continue;
        float v[B];
#pragma unroll
        for (int i = 0; i < B; ++i) v[i] = lt[rb * B + i][cc];
        quant_store<B, NV>(v, s_t, tcodes + col * (m / 2) + row / 2, tscales + col * (m / B) + row / B);
      }
    }
    METIS_LDS_BARRIER();  // the tile's LDS is free for the next one
  };
  Pre pre0, pre1;
  load_pre(p0, pre0);
  // pairs of tiles, then an odd one: no exit between the two tiles of a
  // pair, which would leave the waits at the loop head uncounted
  int p = p0;
  for (; p + 1 < p1; p += 2) {
    tile(p, pre0, pre1);
    tile(p + 1, pre1, pre0);
  }
  if (p < p1) tile(p, pre0, pre1);
  if (AMAX_ONLY) {
    mx = wave_max(mx);
    if (lane == 0) atomicMax(amax, __float_as_uint(mx));
  }
}

// ==================================================================== host
template <typename T, bool MEAN>
metis_status_t run_factors_and_residual(const SplitPlan &p, const T *A, int64_t lda, metis_split_t *out,
                                        const float *mu, hipStream_t st);

// The sketch and the projection with the exact count of 16-column tiles
// compiled in for the common sketch widths (lp = 80, 96: one tile of kLpMax
// columns), else the form that tests the count at run time.
template <typename T, bool HL>
void launch_sketch(dim3 grid, hipStream_t st, const T *A, int64_t m, int64_t n, int64_t lda,
                   const unsigned short *omt, int l, int lp, int64_t chunk, float *ysk) {
  if (lp == 80)
    sketch_kernel<T, HL, kSketchRS, 5><<<grid, kThreads, 0, st>>>(A, m, n, lda, omt, l, lp, chunk, ysk);
  else if (lp == 96)
    sketch_kernel<T, HL, kSketchRS, 6><<<grid, kThreads, 0, st>>>(A, m, n, lda, omt, l, lp, chunk, ysk);
  else
    sketch_kernel<T, HL><<<grid, kThreads, 0, st>>>(A, m, n, lda, omt, l, lp, chunk, ysk);
}

template <typename T>
void launch_project(dim3 grid, hipStream_t st, const T *A, int64_t m, int64_t n, int64_t lda,
                    const unsigned short *qt, int l, int lp, int64_t chunk_rows, float *btp) {
  if (lp == 80)
    project_kernel<T, 5><<<grid, kThreads, 0, st>>>(A, m, n, lda, qt, l, lp, chunk_rows, btp);
  else if (lp == 96)
    project_kernel<T, 6><<<grid, kThreads, 0, st>>>(A, m, n, lda, qt, l, lp, chunk_rows, btp);
  else
    project_kernel<T><<<grid, kThreads, 0, st>>>(A, m, n, lda, qt, l, lp, chunk_rows, btp);
}

template <typename T>
metis_status_t run_split(const SplitPlan &p, const T *A, int64_t lda, const void *omega, metis_split_t *out,
                         int32_t *info, hipStream_t st) {
  const int64_t m = p.m, n = p.n;
  const int l = p.l, lp = p.lp, k = p.k, kp = p.kp;
  const bool nv = p.fmt == METIS_NVFP4;
  const unsigned lz = (unsigned)cdiv(lp, kLpMax);  // sketch-column tiles
  // ---- pass 1: sketch
  const float *ysrc;
  int yparts;
  if (p.kind == METIS_OMEGA_GAUSSIAN) {
    omega_transpose_kernel<<<(unsigned)cdiv(n, kOtRows), 256, 0, st>>>((const unsigned short *)omega, n, l, lp,
                                                                       p.omt);
    launch_sketch<T, false>(dim3((unsigned)cdiv(m, 64 * kSketchRS), p.sk, lz), st, A, m, n, lda, p.omt, l, lp,
                            p.sk_chunk, p.ysk);
    ysrc = p.ysk;
    yparts = p.sk;
  } else {
    gather_kernel<T><<<(unsigned)cdiv(m * l, 256), 256, 0, st>>>(A, m, n, lda, (const int *)omega, l, p.ysk);
    ysrc = p.ysk;
    yparts = 1;
  }
  const unsigned rgrid_red = (unsigned)cdiv(lp * lp, 32);  // 8 lanes per element
  if (!p.wide) {
    // ---- CholeskyQR2 (LDS-resident small matrices) of the sketch's sum of
    // parts: Q (m x l) and its bf16 hi/lo transpose
    auto cholqr2_y = [&](const float *src, int parts) {
      gram_kernel<<<p.gy_parts, kGramThreads, 0, st>>>(src, parts, m * l, m, l, lp, nullptr,
                                                       parts > 1 ? p.y : nullptr, nullptr, p.gpart);
      const float *y = parts > 1 ? p.y : src;
      gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gy_parts, lp * lp, p.gram);
      chol_small_kernel<<<1, kCholThreads, 0, st>>>(p.gram, l, lp, p.rinv, info ? info : p.info_ws);
      gram_kernel<<<p.gy_parts, kGramThreads, 0, st>>>(y, 1, 0, m, l, lp, p.rinv, p.q1, nullptr, p.gpart);
      gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gy_parts, lp * lp, p.gram);
      chol_small_kernel<<<1, kCholThreads, 0, st>>>(p.gram, l, lp, p.rinv, p.info_ws);
      gram_kernel<<<p.gy_parts, kGramThreads, 0, st>>>(p.q1, 1, 0, m, l, lp, p.rinv, p.q, p.qt, nullptr);
    };
    cholqr2_y(ysrc, yparts);
    // ---- power iterations: Z = orth(A^T Q) by CholeskyQR2 over the n rows,
    // then Y = A Z (Z as bf16 hi + lo) and Q = orth(Y) again
    for (int it = 0; it < p.power; ++it) {
      launch_project<T>(dim3((unsigned)cdiv(n, 128), p.pk, lz), st, A, m, n, lda, p.qt, l, lp, p.pk_rows, p.btp);
      sum_parts4_kernel<<<(unsigned)cdiv(n * l, 1024), 256, 0, st>>>(p.btp, p.pk, n * l, n * l, p.bt);
      gram_kernel<<<p.gb_parts, kGramThreads, 0, st>>>(p.bt, 1, 0, n, l, lp, nullptr, nullptr, nullptr, p.gpart);
      gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gb_parts, lp * lp, p.gram);
      chol_small_kernel<<<1, kCholThreads, 0, st>>>(p.gram, l, lp, p.rinv, p.info_ws);
      gram_kernel<<<p.gb_parts, kGramThreads, 0, st>>>(p.bt, 1, 0, n, l, lp, p.rinv, p.z1, nullptr, p.gpart);
      gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gb_parts, lp * lp, p.gram);
      chol_small_kernel<<<1, kCholThreads, 0, st>>>(p.gram, l, lp, p.rinv, p.info_ws);
      gram_kernel<<<p.gb_parts, kGramThreads, 0, st>>>(p.z1, 1, 0, n, l, lp, p.rinv, nullptr, p.zt, nullptr);
      launch_sketch<T, true>(dim3((unsigned)cdiv(m, 64 * kSketchRS), p.sk, lz), st, A, m, n, lda, p.zt, l, lp,
                             p.sk_chunk, p.ysk);
      cholqr2_y(p.ysk, p.sk);
    }
    // ---- pass 2: projection B^T = A^T Q, then the Gram B B^T
    launch_project<T>(dim3((unsigned)cdiv(n, 128), p.pk, lz), st, A, m, n, lda, p.qt, l, lp, p.pk_rows, p.btp);
    sum_parts4_kernel<<<(unsigned)cdiv(n * l, 1024), 256, 0, st>>>(p.btp, p.pk, n * l, n * l, p.bt);
    gram_kernel<<<p.gb_parts, kGramThreads, 0, st>>>(p.bt, 1, 0, n, l, lp, nullptr, nullptr, nullptr, p.gpart);
    gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gb_parts, lp * lp, p.gram);
  } else {
    // ---- the same steps with the l x l matrices in global scratch
    const float *y = ysrc;
    if (yparts > 1) {
      sum_parts_kernel<<<(unsigned)cdiv(m * l, 256), 256, 0, st>>>(ysrc, yparts, m * l, m * l, p.y);
      y = p.y;
    }
    const unsigned nt = (unsigned)(lp / 64);
    gram_tile_kernel<<<dim3(p.gy_parts, nt, nt), kThreads, 0, st>>>(y, m, l, lp, p.gy_rows, p.gpart);
    gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gy_parts, lp * lp, p.gram);
    metis_status_t ws = metis_wide::wide_chol_inv(p.gram, l, lp, p.rinv, info ? info : p.info_ws, p.wa, p.winv,
                                                  p.waux, st);
    if (ws != METIS_OK) return ws;
    apply_rinv_kernel<<<dim3((unsigned)cdiv(m, 64), nt), kThreads, 0, st>>>(y, m, l, lp, p.rinv, p.q1, nullptr);
    gram_tile_kernel<<<dim3(p.gy_parts, nt, nt), kThreads, 0, st>>>(p.q1, m, l, lp, p.gy_rows, p.gpart);
    gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gy_parts, lp * lp, p.gram);
    ws = metis_wide::wide_chol_inv(p.gram, l, lp, p.rinv, p.info_ws, p.wa, p.winv, p.waux, st);
    if (ws != METIS_OK) return ws;
    apply_rinv_kernel<<<dim3((unsigned)cdiv(m, 64), nt), kThreads, 0, st>>>(p.q1, m, l, lp, p.rinv, p.q, p.qt);
    launch_project<T>(dim3((unsigned)cdiv(n, 128), p.pk, lz), st, A, m, n, lda, p.qt, l, lp, p.pk_rows, p.btp);
    const float *bt = p.btp;
    if (p.pk > 1) {
      sum_parts_kernel<<<(unsigned)cdiv(n * l, 256), 256, 0, st>>>(p.btp, p.pk, n * l, n * l, p.bt);
      bt = p.bt;
    }
    gram_tile_kernel<<<dim3(p.gb_parts, nt, nt), kThreads, 0, st>>>(bt, n, l, lp, p.gb_rows, p.gpart);
    gram_reduce_kernel<<<rgrid_red, 256, 0, st>>>(p.gpart, p.gb_parts, lp * lp, p.gram);
  }
  // ---- small SVD of B (from its Gram, in p.gram) and the factors
  if (!p.wide) {
    if (lp == 80)
      tridiag_kernel<2, 20><<<1, kTriThreads, 0, st>>>(p.gram, l, lp, p.waux, p.waux + lp, p.waux + 2 * lp, p.wv);
    else if (lp > 64)
      tridiag_kernel<2><<<1, kTriThreads, 0, st>>>(p.gram, l, lp, p.waux, p.waux + lp, p.waux + 2 * lp, p.wv);
    else
      tridiag_kernel<1><<<1, kTriThreads, 0, st>>>(p.gram, l, lp, p.waux, p.waux + lp, p.waux + 2 * lp, p.wv);
    const metis_status_t es = metis_wide::eigh_tridiag(l, lp, k, p.wv, p.evec, p.sig_inv, out->S, p.wa, p.waux, st);
    if (es != METIS_OK) return es;
    assemble_u_kernel<<<p.am_parts, kThreads, 0, st>>>(p.q, m, l, lp, k, p.evec, p.am_rows, out->U, p.am_val,
                                                       p.am_idx);
    assemble_v_kernel<<<(unsigned)cdiv(n, asm_chunk_rows(k)), kThreads, 0, st>>>(p.bt, n, l, lp, k, p.evec,
                                                                                 p.sig_inv, out->V);
  } else {
    const float *bt = p.pk > 1 ? p.bt : p.btp;
    const metis_status_t es =
        metis_wide::wide_eigh(p.gram, l, lp, k, p.evec, p.sig_inv, out->S, p.wg, p.wv, p.wa, p.waux, st);
    if (es != METIS_OK) return es;
    metis_status_t as = metis_wide::wide_assemble(p.q, m, l, lp, k, p.evec, nullptr, out->U, p.am_val, p.am_idx, st);
    if (as == METIS_OK)
      as = metis_wide::wide_assemble(bt, n, l, lp, k, p.evec, p.sig_inv, out->V, nullptr, nullptr, st);
    if (as != METIS_OK) return as;
  }
  sign_kernel<<<1, 1024, 0, st>>>(p.am_val, p.am_idx, p.am_parts, k, p.sign);
  return run_factors_and_residual<T, false>(p, A, lda, out, nullptr, st);
}

// Factor quantization (signs applied from p.sign) and the residual pass,
// shared by the spectral and the mean-residual splits.
template <typename T, bool MEAN>
metis_status_t run_factors_and_residual(const SplitPlan &p, const T *A, int64_t lda, metis_split_t *out,
                                        const float *mu, hipStream_t st) {
  const int64_t m = p.m, n = p.n;
  const int k = p.k, kp = p.kp;
  const bool nv = p.fmt == METIS_NVFP4;
  const int B = nv ? 16 : 32;
  const unsigned fgrid = (unsigned)cdiv(std::max(m, n) / B * kp, kThreads);
  if (nv) {
    fill_u32<<<1, 64, 0, st>>>(p.amax, 0u, 8);
    amax_f32_kernel<<<64, 256, 0, st>>>(out->U, m, k, p.amax + 0);
    amax_f32_kernel<<<64, 256, 0, st>>>(out->V, n, k, p.amax + 1);
    factor_kernel<true><<<dim3(fgrid, 2), kThreads, 0, st>>>(
        out->U, out->V, m, n, k, kp, p.sign, out->S, out->Ut_q.codes, out->Ut_q.scales, out->Ut_q.tensor_scale,
        out->Vt_q.codes, out->Vt_q.scales, out->Vt_q.tensor_scale, p.amax, p.uhl, p.whl);
  } else {
    factor_kernel<false><<<dim3(fgrid, 2), kThreads, 0, st>>>(
        out->U, out->V, m, n, k, kp, p.sign, out->S, out->Ut_q.codes, out->Ut_q.scales, nullptr, out->Vt_q.codes,
        out->Vt_q.scales, nullptr, p.amax, p.uhl, p.whl);
  }
  // ---- pass 3: residual + quantization (NVFP4: a max pass first)
  // persistent residual: groups of eight workgroups, up to eight groups per
  // XCD (two resident workgroups per CU; registers bound it)
  const int64_t nblk = (cdiv(m, kRT) + 1) / 2 * cdiv(cdiv(n, kRC), 4);
  const unsigned rgrid = (unsigned)(kResGroup * kXcds * std::min<int64_t>(8, cdiv(nblk, kXcds)));
  auto launch = [&](auto kpc) {
    constexpr int KP = decltype(kpc)::value;
    if (nv) {
      residual_kernel<T, true, true, MEAN, KP><<<rgrid, kThreads, 0, st>>>(
          A, m, n, lda, p.uhl, p.whl, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, p.amax + 2, mu);
      residual_kernel<T, true, false, MEAN, KP><<<rgrid, kThreads, 0, st>>>(
          A, m, n, lda, p.uhl, p.whl, out->R_q.codes, out->R_q.scales, out->R_q.tensor_scale, out->Rt_q.codes,
          out->Rt_q.scales, out->Rt_q.tensor_scale, p.amax + 2, mu);
    } else {
      residual_kernel<T, false, false, MEAN, KP><<<rgrid, kThreads, 0, st>>>(
          A, m, n, lda, p.uhl, p.whl, out->R_q.codes, out->R_q.scales, nullptr, out->Rt_q.codes, out->Rt_q.scales,
          nullptr, nullptr, mu);
    }
  };
  // the mean split reads no factor panels: one instance serves it
  if (MEAN || kp == 32) launch(std::integral_constant<int, 32>{});
  else if (kp == 64) launch(std::integral_constant<int, 64>{});
  else if (kp == 96) launch(std::integral_constant<int, 96>{});
  else return METIS_ERR_INVALID;
  METIS_LAUNCH_CHECK();
  return METIS_OK;
}

// ------------------------------------------------------- mean-residual split
// Mean over all rows of A (Averis, "Averaging-Induced Residual Splitting",
// as retold on the zhu318.com page, method paragraphs), as a rank-1 split
// record: U = 1, S = 1, V = mu. Column sums run in fp64, rows in order: chunk
// c of rows is summed per column (16 bytes of columns per thread, eight rows'
// loads in flight), then the chunks in order.
constexpr int kMeanChunkRows = 128;

template <typename T>
__global__ void __launch_bounds__(256)
    colsum_kernel(const T *__restrict__ A, int64_t m, int64_t n, int64_t lda, double *__restrict__ part) {
  constexpr int V = 16 / (int)sizeof(T);  // columns per thread
  const int64_t j0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  const int c = blockIdx.y;
  if (j0 >= n) return;
  const int64_t r0 = (int64_t)c * kMeanChunkRows, r1 = std::min<int64_t>(m, r0 + kMeanChunkRows);
  double s[V];
#pragma unroll
  for (int v = 0; v < V; ++v) s[v] = 0.0;
  int64_t r = r0;
  for (; r + 8 <= r1; r += 8) {
    uint4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *(const uint4 *)(A + (r + u) * lda + j0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const T *e = (const T *)&x[u];
#pragma unroll
      for (int v = 0; v < V; ++v) s[v] += (double)load_f32(e + v);
    }
  }
  for (; r < r1; ++r) {
    const uint4 x = *(const uint4 *)(A + r * lda + j0);
    const T *e = (const T *)&x;
#pragma unroll
    for (int v = 0; v < V; ++v) s[v] += (double)load_f32(e + v);
  }
#pragma unroll
  for (int v = 0; v < V; ++v) part[(int64_t)c * n + j0 + v] = s[v];
}

// mu = (sum of the chunk sums in order) / m into V; U = 1, S = 1, sign = 1.
__global__ void mean_finish_kernel(const double *__restrict__ part, int chunks, int64_t m, int64_t n,
                                   float *__restrict__ V, float *__restrict__ U, float *__restrict__ S,
                                   float *__restrict__ sign) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    double s = 0.0;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * n + i];
    V[i] = (float)(s / (double)m);
  }
  if (i < m) U[i] = 1.0f;
  if (i == 0) {
    S[0] = 1.0f;
    sign[0] = 1.0f;
  }
}

struct MeanPlan {
  SplitPlan sp;  // the fields the factor and residual passes use
  double *part;  // chunks x n
  int chunks;
  size_t bytes;
};

MeanPlan make_mean_plan(int64_t m, int64_t n, int fmt, int elem, void *ws) {
  MeanPlan p{};
  p.sp.m = m; p.sp.n = n; p.sp.l = 1; p.sp.lp = 16; p.sp.k = 1; p.sp.kp = 32;
  p.sp.fmt = fmt; p.sp.elem = elem; p.sp.wide = false; p.sp.kind = -1;
  p.chunks = (int)cdiv(m, kMeanChunkRows);
  metis_host::Carver c(ws);
  p.part = c.take<double>((size_t)p.chunks * n);
  p.sp.sign = c.take<float>(1);
  p.sp.uhl = c.take<unsigned short>((size_t)2 * m * p.sp.kp);
  p.sp.whl = c.take<unsigned short>((size_t)2 * n * p.sp.kp);
  p.sp.amax = c.take<uint32_t>(8);
  p.bytes = c.bytes();
  p.sp.bytes = p.bytes;
  return p;
}

template <typename T>
metis_status_t run_mean_split(const MeanPlan &p, const T *A, int64_t lda, metis_split_t *out, hipStream_t st) {
  const int64_t m = p.sp.m, n = p.sp.n;
  constexpr int V = 16 / (int)sizeof(T);
  colsum_kernel<T><<<dim3((unsigned)cdiv(n, 256 * V), (unsigned)p.chunks), 256, 0, st>>>(A, m, n, lda, p.part);
  mean_finish_kernel<<<(unsigned)cdiv(std::max(m, n), 256), 256, 0, st>>>(p.part, p.chunks, m, n, out->V, out->U,
                                                                           out->S, p.sp.sign);
  return run_factors_and_residual<T, true>(p.sp, A, lda, out, out->V, st);
}

bool fp4_ok(const metis_fp4_t &q, int fmt, bool need_ts) {
  return q.codes && q.scales && q.fmt == fmt && (((uintptr_t)q.codes) & 15) == 0 && (!need_ts || q.tensor_scale);
}

}  // namespace

extern "C" size_t metis_split_power_workspace_bytes(int64_t m, int64_t n, int32_t l, int32_t k, metis_omega_t kind,
                                                    int32_t q, metis_fmt_t fmt) {
  if (m <= 0 || n <= 0 || l <= 0 || k <= 0 || q < 0) return 0;
  // the plan depends on the element size; cover both input types
  return std::max(make_plan(m, n, l, k, kind, fmt, 4, nullptr, q).bytes,
                  make_plan(m, n, l, k, kind, fmt, 2, nullptr, q).bytes);
}

extern "C" size_t metis_split_workspace_bytes(int64_t m, int64_t n, int32_t l, int32_t k, metis_omega_t kind,
                                              metis_fmt_t fmt) {
  return metis_split_power_workspace_bytes(m, n, l, k, kind, 0, fmt);
}

namespace {
// Argument checks and the plan of a split (q power iterations).
metis_status_t split_entry(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda, const void *omega,
                           metis_omega_t kind, int32_t l, int32_t k, int32_t q, metis_fmt_t fmt, metis_split_t *out,
                           int32_t *info, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (q < 0) return METIS_ERR_INVALID;
  if (q > kMaxPowerIterations || (q > 0 && l > kLpMax)) return METIS_ERR_UNSUPPORTED;
  if (!A || !omega || !out) return METIS_ERR_INVALID;
  if (dt != METIS_F32 && dt != METIS_BF16) return METIS_ERR_INVALID;
  if (fmt != METIS_MXFP4 && fmt != METIS_NVFP4) return METIS_ERR_INVALID;
  if (kind != METIS_OMEGA_GAUSSIAN && kind != METIS_OMEGA_COLUMNS) return METIS_ERR_INVALID;
  if (m <= 0 || n <= 0 || m % 32 || n % 32 || lda < n) return METIS_ERR_INVALID;
  if (k < 1 || l < k || l > m || l > n) return METIS_ERR_INVALID;
  const int elem = dt == METIS_F32 ? 4 : 2;
  if (((uintptr_t)A) & 15 || (lda * elem) % 16) return METIS_ERR_INVALID;
  if (l > 512) return METIS_ERR_UNSUPPORTED;
  if (k > 96) return METIS_ERR_UNSUPPORTED;
  if (!out->U || !out->S || !out->V) return METIS_ERR_INVALID;
  const bool nv = fmt == METIS_NVFP4;
  if (!fp4_ok(out->Ut_q, fmt, nv) || !fp4_ok(out->Vt_q, fmt, nv)) return METIS_ERR_INVALID;
  const bool want_n = out->R_q.codes != nullptr, want_t = out->Rt_q.codes != nullptr;
  if (want_n && !fp4_ok(out->R_q, fmt, nv)) return METIS_ERR_INVALID;
  if (want_t && !fp4_ok(out->Rt_q, fmt, nv)) return METIS_ERR_INVALID;
  if (!ws) return METIS_ERR_WORKSPACE;
  if (((uintptr_t)ws) & 255) return METIS_ERR_INVALID;
  SplitPlan p = make_plan(m, n, l, k, kind, fmt, elem, ws, q);
  if (ws_bytes < p.bytes) return METIS_ERR_WORKSPACE;
  out->m = m;
  out->n = n;
  out->k = k;
  out->Ut_q.rows = k; out->Ut_q.cols = m;
  out->Vt_q.rows = k; out->Vt_q.cols = n;
  out->R_q.rows = m; out->R_q.cols = n;
  out->Rt_q.rows = n; out->Rt_q.cols = m;
  if (dt == METIS_F32) return run_split<float>(p, (const float *)A, lda, omega, out, info, stream);
  return run_split<unsigned short>(p, (const unsigned short *)A, lda, omega, out, info, stream);
}
}  // namespace

extern "C" metis_status_t metis_split_power(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                                            const void *omega, metis_omega_t kind, int32_t l, int32_t k, int32_t q,
                                            metis_fmt_t fmt, metis_split_t *out, int32_t *info, void *ws,
                                            size_t ws_bytes, hipStream_t stream) {
  return split_entry(A, dt, m, n, lda, omega, kind, l, k, q, fmt, out, info, ws, ws_bytes, stream);
}

extern "C" metis_status_t metis_split(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                                      const void *omega, metis_omega_t kind, int32_t l, int32_t k, metis_fmt_t fmt,
                                      metis_split_t *out, int32_t *info, void *ws, size_t ws_bytes,
                                      hipStream_t stream) {
  return metis_split_power(A, dt, m, n, lda, omega, kind, l, k, 0, fmt, out, info, ws, ws_bytes, stream);
}

extern "C" size_t metis_mean_split_workspace_bytes(int64_t m, int64_t n, metis_fmt_t fmt) {
  if (m <= 0 || n <= 0) return 0;
  return make_mean_plan(m, n, fmt, 2, nullptr).bytes;
}

extern "C" metis_status_t metis_mean_split(const void *A, metis_dtype_t dt, int64_t m, int64_t n, int64_t lda,
                                           metis_fmt_t fmt, metis_split_t *out, void *ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (!A || !out) return METIS_ERR_INVALID;
  if (dt != METIS_F32 && dt != METIS_BF16) return METIS_ERR_INVALID;
  if (fmt != METIS_MXFP4 && fmt != METIS_NVFP4) return METIS_ERR_INVALID;
  if (m <= 0 || n <= 0 || m % 32 || n % 32 || lda < n) return METIS_ERR_INVALID;
  const int elem = dt == METIS_F32 ? 4 : 2;
  if (((uintptr_t)A) & 15 || (lda * elem) % 16) return METIS_ERR_INVALID;
  if (!out->U || !out->S || !out->V) return METIS_ERR_INVALID;
  const bool nv = fmt == METIS_NVFP4;
  if (!fp4_ok(out->Ut_q, fmt, nv) || !fp4_ok(out->Vt_q, fmt, nv)) return METIS_ERR_INVALID;
  if (out->R_q.codes && !fp4_ok(out->R_q, fmt, nv)) return METIS_ERR_INVALID;
  if (out->Rt_q.codes && !fp4_ok(out->Rt_q, fmt, nv)) return METIS_ERR_INVALID;
  if (!ws) return METIS_ERR_WORKSPACE;
  if (((uintptr_t)ws) & 255) return METIS_ERR_INVALID;
  MeanPlan p = make_mean_plan(m, n, fmt, elem, ws);
  if (ws_bytes < p.bytes) return METIS_ERR_WORKSPACE;
  out->m = m;
  out->n = n;
  out->k = 1;
  out->Ut_q.rows = 1; out->Ut_q.cols = m;
  out->Vt_q.rows = 1; out->Vt_q.cols = n;
  out->R_q.rows = m; out->R_q.cols = n;
  out->Rt_q.rows = n; out->Rt_q.cols = m;
  if (dt == METIS_F32) return run_mean_split<float>(p, (const float *)A, lda, out, stream);
  return run_mean_split<unsigned short>(p, (const unsigned short *)A, lda, out, stream);
}
