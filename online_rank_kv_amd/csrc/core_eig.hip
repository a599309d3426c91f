// Symmetric eigensolver for the merge core Z^T Z = diag(sigma^2, 0) + M^T M
// and for the re-orthogonalisation matrix (iS-KV notes §4.2 / §4.4 need the
// top singular triplets of the small core; its size does not grow with n).
//
// gfx950 design. At r = 256, b = 32 the core is 288 x 288: a single-workgroup
// Jacobi cannot keep it in 160 KB of LDS and takes tens of ms through L2. The
// core is, however, nearly diagonal after the first merges (old directions
// are decoupled up to O(b/n)), so it is solved by a parallel refinement of
// the eigenvector matrix W (initially I), every step run on many workgroups:
//   S = W^T A W                                   (two fp64 GEMMs)
//   pairs with |s_ij| > omega |s_jj - s_ii| ("strongly coupled", near ties)
//     form connected clusters; clusters of <= 6 indices are diagonalised
//     exactly by a small cyclic Jacobi, larger ones get exact 2x2 rotations
//     on a greedy matching of their strong pairs;          (one workgroup)
//   every other pair gets the first-order Jacobi angle
//     K_ij = s_ij / (s_jj - s_ii) (K antisymmetric, clipped),
//   W <- W R X with X = I + K (I + K/2), the exponential of K to second
//   order                                           (two GEMMs)
//   W <- 1.5 W - 0.5 W (W^T W) (Newton-Schulz, two GEMMs) before the next S
// until every scaled coupling |s_ij| / sqrt(s_ii s_jj) is below the
// tolerance. This is the first-order eigenvector refinement of the Jacobi
// family (all rotations of a sweep at once), with near-ties handled exactly.
// A final Newton-Schulz step restores W^T W = I. Cores that do not converge
// in PCJ_MAXIT steps (strongly mixed early merges) fall back to the
// single-workgroup cyclic Jacobi.
//
// Tolerance. isvd_sym_eig asks for eigenvectors to 1e-10 in the scaled
// coupling |s_ij| / sqrt(s_ii s_jj), which holds the smallest eigenvectors to
// the same relative accuracy as the largest. A merge only needs the product
// C B^T: rotations among kept directions leave it unchanged, and a rotation
// left between a kept and a dropped direction, or among kept directions
// through the stored sigma (the next merge takes C^T C as diagonal), moves
// it by about |s_ij| / sqrt(max(s_ii, s_jj) s_max) relative to its largest
// singular value (coupling_at). Merges and re-orthogonalisations stop when
// that measure is below 1e-8, far below the fp32 rounding the factors carry.
// On the 16K-row K and V streams the scaled measure is held up for two more
// steps by pairs between a large direction and one of the smallest ones
// (scaled coupling ~3e-3 after the first step where the product measure is
// ~1e-5), which do not change the product.
#include "iskv_internal.h"

#include <math.h>

namespace {

#ifndef ISKV_PCJ_MAXIT
#define ISKV_PCJ_MAXIT 6
#endif
constexpr int PCJ_MAXIT = ISKV_PCJ_MAXIT;
constexpr double PCJ_OMEGA = 0.1;
constexpr double PCJ_CLIP = 0.2;
constexpr int CMAX_S = ISKV_PCJ_CMAX;  // largest cluster diagonalised exactly
constexpr int NCL_MAX = 64;    // clusters handled exactly per step
constexpr int EMAX = ISKV_PCJ_EMAX;  // strong pairs recorded per step
constexpr int NPAIR_MAX = 512; // matched pairs per step

constexpr int FLAG_CONV = 1;
constexpr int FLAG_FALLBACK = 2;
constexpr int FLAG_COLD = 4;     // the fallback starts from A itself
constexpr int FLAG_NS = 16;      // converged, but W needs the final Newton-Schulz step

// ----------------------------------------------------------------------------
// C = alpha * opA(A) opB(B) + beta * Cin + gamma * I, all m x m (m from
// st[ST_JM]), fp64 on the matrix cores: a workgroup of four waves owns a
// 32 x 32 output tile, each wave a 16 x 16 block accumulated with
// V_MFMA_F64_16X16X4F64 (A fragment: lane l holds A[l % 16][l / 16]; B
// fragment: lane l holds B[l / 16][l % 16]; result: lane l, element e holds
// C[l / 16 + 4 e][l % 16], as measured on gfx950). Operand tiles of 32 x 16
// are staged in LDS.
// mode 0: skip the launch when (st[ST_PCJ] & FLAG_CONV).
// mode 1: when converged, copy Cin (the current W) to C instead.
// mode 2: always run.
// mode 3: run only when the refinement has not converged.
// mode 4 (paired products): skip when it converged at a step >= 1 whose W,
//   already orthonormalised with A W formed, came from an iterate within
//   1e-4 of orthonormal (FLAG_NS clear); run after step 0, without
//   convergence, or with FLAG_NS.
typedef double v4d __attribute__((ext_vector_type(4)));
// Branch-free masking of a loaded value: the bits are ANDed with 0 or
// all-ones, so the load itself is never placed under a branch and every load
// of a panel can be in flight at once.
__device__ __forceinline__ double keep_if(double v, bool keep) {
  return __longlong_as_double(__double_as_longlong(v) & -(long long)keep);
}

// fp64 GEMM on the matrix cores (v_mfma_f64_16x16x4f64) for the core
// eigensolver:  C = alpha op(A) op(B) + beta Cin + gamma I  over the m x m
// leading block (m = st[ST_JM]), op = transpose when TA / TB.
// One 16 x 16 output tile per 256-thread workgroup; its 4 waves split the
// depth in chunks of 16 (wave w takes chunks w, w+4, ...), load their
// operands straight from global memory into registers (no LDS staging), and
// the four partial tiles are summed through LDS. Inside a chunk, lane l
// (row or column l%16, group g = l/16) takes depths 16 c + 4 g + q for MFMA
// step q, so that the operands stored along k are contiguous per lane.
// Matrices have a leading dimension that is a multiple of 16 and at least
// m_max rounded up to 16, so every index of a 16-chunk that starts below m
// lies in the allocation: entries with depth >= m are zeroed, rows and
// columns >= m of a tile that starts below m are computed and dropped.
constexpr int DG_CH = 5;   // chunks per wave kept in flight (m <= 320 in one pass)
constexpr int DG2_NW = 4;  // waves of the paired GEMM (a depth split 8 ways measured slower)

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void dgemm_kernel(const double* __restrict__ A, int lda,
                                                    const double* __restrict__ B, int ldb, double* C,
                                                    int ldc, const double* Cin, int ldcin,
                                                    double alpha, double beta, double gamma,
                                                    const int32_t* __restrict__ st, int mode,
                                                    int m_max,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A = iskv_rb(A, bdel);
  B = iskv_rb(B, bdel);
  C = iskv_rb(C, bdel);
  Cin = iskv_rb(Cin, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  (void)m_max;
  double av[DG_CH][4], bv[DG_CH][4];
  // A(i0 + r, k) and B(k, j0 + r) for k = 16 c + 4 g + q
  auto load = [&](int u, int c) {
    const int kb = 16 * c + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[u][q] = TA ? A[(size_t)(kb + q) * lda + i0 + r] : A[(size_t)(i0 + r) * lda + kb + q];
      bv[u][q] = TB ? B[(size_t)(j0 + r) * ldb + kb + q] : B[(size_t)(kb + q) * ldb + j0 + r];
    }
  };
  // the state is read before any operand load: a launch skipped because
  // the refinement has converged (or a tile beyond m) moves no data
  const int m = st[ST_JM];
  if (i0 >= m || j0 >= m) return;
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  if ((mode == 0 || mode == 3) && conv) return;
  if (mode == 1 && conv) {
    const int i = i0 + (t >> 4), j = j0 + (t & 15);
    if (i < m && j < m) C[(size_t)i * ldc + j] = Cin[(size_t)i * ldcin + j];
    return;
  }
  const int nch = (m + 15) / 16;
#pragma unroll
  for (int u = 0; u < DG_CH; ++u)
    if (wave + 4 * u < nch) load(u, wave + 4 * u);
  v4d acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = wave; c0 < nch; c0 += 4 * DG_CH) {
    if (c0 != wave) {
#pragma unroll
      for (int u = 0; u < DG_CH; ++u)
        if (c0 + 4 * u < nch) load(u, c0 + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < DG_CH; ++u) {
      const int c = c0 + 4 * u;
      if (c < nch) {
        const int kb = 16 * c + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool in = kb + q < m;
          const double a = keep_if(av[u][q], in), bb = keep_if(bv[u][q], in);
          if (q & 1) acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc2, 0, 0, 0);
          else acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc, 0, 0, 0);
        }
      }
    }
  }
  acc += acc2;
  __shared__ double red[3][4][64];
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave > 0) return;
  // result lane l, element e is D(l/16 + 4e, l%16)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + g + 4 * e, j = j0 + r;
    if (i < m && j < m) {
      double o = alpha * (acc[e] + red[0][e][lane] + red[1][e][lane] + red[2][e][lane]);
      if (beta != 0.0) o += beta * Cin[(size_t)i * ldcin + j];
      if (i == j) o += gamma;
      C[(size_t)i * ldc + j] = o;
    }
  }
}

template <bool TA, bool TB>
void dgemm(hipStream_t s, int m_max, const double* A, const double* B, double* C, const double* Cin,
           int ld, double alpha, double beta, double gamma, const int32_t* st, int mode,
           const int64_t* bd, int bc) {
  dim3 grid((m_max + 15) / 16, (m_max + 15) / 16);
  hipLaunchKernelGGL((dgemm_kernel<TA, TB>), bz(grid, bc), dim3(256), 0, s, A, ld, B, ld, C, ld, Cin, ld, alpha,
                     beta, gamma, st, mode, m_max, bd);
}

// Scaled coupling |s_ij| / sqrt(s_ii s_jj). A non-finite entry counts as an
// infinite coupling: the maxima are taken with fmax, which would drop a NaN,
// and a NaN must never pass the convergence test (it sends the solve to the
// fallback from A itself).
__device__ __forceinline__ double coupling(double sij, double di, double dj) {
  if (!isfinite(sij) || !isfinite(di) || !isfinite(dj)) return INFINITY;
  double dd = di * dj;
  double a = fabs(sij);
  if (dd > 0.0) return a / sqrt(dd);
  return a > 0.0 ? INFINITY : 0.0;
}

// The coupling a step measures. With sref = 0: the scaled coupling above,
// which asks every eigenvector, the smallest included, for the tolerance
// (isvd_sym_eig, the refit). With sref > 0 (the largest diagonal entry of the
// matrix being solved; merges and re-orthogonalisations) it measures how far
// the pair's remaining rotation moves the represented product, relative to
// its largest singular value sigma_1 = sqrt(sref):
//   * directions on the same side of the truncation (both kept or both
//     dropped): a rotation between them leaves the product unchanged, and
//     the coupling itself, dropped from the stored sigma (the next merge
//     takes C^T C as diagonal), moves it by
//       |s_ij| / sqrt(max(|s_ii|, |s_jj|) sref);
//   * a kept and a dropped direction (diagonal values on both sides of dcut,
//     between the keep-th and (keep+1)-th largest diagonal entries of the
//     matrix): the rotation angle min(1, |s_ij| / |s_jj - s_ii|) weighted by
//     sqrt(max(|s_ii|, |s_jj|) / sref), the larger of the two.
// dcut < 0: nothing is dropped. A pair of one large and one of the smallest
// directions then counts by sigma_j / sigma_1 less than its scaled coupling,
// so such pairs no longer hold a merge's core for extra steps, while a
// near-tie across the truncation still has to be resolved.
__device__ __forceinline__ double coupling_at(double sij, double di, double dj, double sref, double dcut) {
  if (!(sref > 0.0)) return coupling(sij, di, dj);
  if (!isfinite(sij) || !isfinite(di) || !isfinite(dj)) return INFINITY;
  const double a = fabs(sij);
  if (a == 0.0) return 0.0;
  const double dm = fmax(fabs(di), fabs(dj));
  double c = a / sqrt(dm * sref);
  if (dcut >= 0.0 && (di > dcut) != (dj > dcut)) c = fmax(c, fmin(1.0, a / fabs(dj - di)) * sqrt(dm / sref));
  return c;
}
__device__ __forceinline__ double coupling_ref(const int32_t* st) { return (double)__int_as_float(st[ST_SREF]); }
__device__ __forceinline__ double coupling_cut(const int32_t* st) { return (double)__int_as_float(st[ST_DCUT]); }

// Two products that share the right operand, one 16 x 16 tile of each per
// workgroup (the right-operand panel is loaded once):
//   C1 = alpha1 op(A1) B + beta1 Cin1,   C2 = alpha2 op(A2) B + beta2 Cin2
// over the m x m leading block (m = st[ST_JM]); same depth split, lane
// layout and skip modes as dgemm_kernel (mode 1 copies Cin1 / Cin2 when the
// refinement has converged). With Dp, the workgroup also writes, for each
// column j of its tile, the partial sum over its 16 rows of C1[i][j] C2[i][j]
// to Dp[blockIdx.y][j]; summed over the row blocks this is the diagonal of
// C1^T C2.
template <bool TA1, bool TA2, int NW>
__global__ __launch_bounds__(64 * NW) void dgemm2_kernel(const double* __restrict__ A1, const double* __restrict__ A2,
                                                     const double* __restrict__ B, int ld, double* C1, double* C2,
                                                     const double* Cin1, const double* Cin2, double alpha1,
                                                     double beta1, double alpha2, double beta2, double* Dp,
                                                     const int32_t* __restrict__ st, int mode,
                                                     const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A1 = iskv_rb(A1, bdel);
  A2 = iskv_rb(A2, bdel);
  B = iskv_rb(B, bdel);
  C1 = iskv_rb(C1, bdel);
  C2 = iskv_rb(C2, bdel);
  Cin1 = iskv_rb(Cin1, bdel);
  Cin2 = iskv_rb(Cin2, bdel);
  Dp = iskv_rb(Dp, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m = st[ST_JM];
  if (i0 >= m || j0 >= m) return;
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  if (mode == 0 && conv) return;
  if (mode == 4 && conv && st[ST_PCJIT] > 0 && !(st[ST_PCJ] & FLAG_NS)) return;
  if (mode == 1 && conv) {
    if (t < 256) {
      const int i = i0 + (t >> 4), j = j0 + (t & 15);
      if (i < m && j < m) {
        C1[(size_t)i * ld + j] = Cin1[(size_t)i * ld + j];
        C2[(size_t)i * ld + j] = Cin2[(size_t)i * ld + j];
      }
    }
    return;
  }
  const int nch = (m + 15) / 16;
  double a1v[DG_CH][4], a2v[DG_CH][4], bv[DG_CH][4];
  auto load = [&](int u, int c) {
    const int kb = 16 * c + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a1v[u][q] = TA1 ? A1[(size_t)(kb + q) * ld + i0 + r] : A1[(size_t)(i0 + r) * ld + kb + q];
      a2v[u][q] = TA2 ? A2[(size_t)(kb + q) * ld + i0 + r] : A2[(size_t)(i0 + r) * ld + kb + q];
      bv[u][q] = B[(size_t)(kb + q) * ld + j0 + r];
    }
  };
  v4d acc1 = {0.0, 0.0, 0.0, 0.0}, acc1b = acc1, acc2 = acc1, acc2b = acc1;
  for (int c0 = wave; c0 < nch; c0 += NW * DG_CH) {
#pragma unroll
    for (int u = 0; u < DG_CH; ++u)
      if (c0 + NW * u < nch) load(u, c0 + NW * u);
#pragma unroll
    for (int u = 0; u < DG_CH; ++u) {
      const int c = c0 + NW * u;
      if (c < nch) {
        const int kb = 16 * c + 4 * g;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool in = kb + q < m;
          const double bb = keep_if(bv[u][q], in);
          if (q & 1) {
            acc1b = __builtin_amdgcn_mfma_f64_16x16x4f64(keep_if(a1v[u][q], in), bb, acc1b, 0, 0, 0);
            acc2b = __builtin_amdgcn_mfma_f64_16x16x4f64(keep_if(a2v[u][q], in), bb, acc2b, 0, 0, 0);
          } else {
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(keep_if(a1v[u][q], in), bb, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(keep_if(a2v[u][q], in), bb, acc2, 0, 0, 0);
          }
        }
      }
    }
  }
  acc1 += acc1b;
  acc2 += acc2b;
  __shared__ double red[NW - 1][2][4][64];
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      red[wave - 1][0][e][lane] = acc1[e];
      red[wave - 1][1][e][lane] = acc2[e];
    }
  }
  __syncthreads();
  if (wave > 0) return;
  // result lane l, element e is D(l/16 + 4e, l%16)
  double dsum = 0.0;
  const int j = j0 + r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + g + 4 * e;
    if (i < m && j < m) {
      double s1 = acc1[e], s2 = acc2[e];
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) {
        s1 += red[w][0][e][lane];
        s2 += red[w][1][e][lane];
      }
      double o1 = alpha1 * s1, o2 = alpha2 * s2;
      if (beta1 != 0.0) o1 += beta1 * Cin1[(size_t)i * ld + j];
      if (beta2 != 0.0) o2 += beta2 * Cin2[(size_t)i * ld + j];
      C1[(size_t)i * ld + j] = o1;
      C2[(size_t)i * ld + j] = o2;
      dsum = fma(o1, o2, dsum);
    }
  }
  if (Dp) {
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    if (g == 0) Dp[(size_t)blockIdx.y * ld + j] = dsum;
  }
}

// S = W^T T (one 16 x 16 tile per workgroup, as dgemm_kernel<true, false>)
// with the strong-pair detection of the refinement in its epilogue. S is
// symmetric, so only tiles on or above the diagonal are computed; each value
// is written to both (i, j) and (j, i). The diagonal of S comes from the
// row-block partial sums Dp of the launch that formed W and T (ceil(m / 16)
// blocks), every pair i < j of the tile gets its scaled coupling, strong
// pairs are appended to the edge list and the tile's largest coupling goes
// to aux[tile] (0 for tiles below the diagonal or outside m x m, and after
// convergence, so the maxima never carry values of an earlier step).
__global__ __launch_bounds__(256) void dgemm_s_kernel(const double* __restrict__ W, const double* __restrict__ T,
                                                      int ld, double* S, const double* __restrict__ Dp,
                                                      double* aux, int* edges, int32_t* st, double tol,
                                                      const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  W = iskv_rb(W, bdel);
  T = iskv_rb(T, bdel);
  S = iskv_rb(S, bdel);
  Dp = iskv_rb(Dp, bdel);
  aux = iskv_rb(aux, bdel);
  edges = iskv_rb(edges, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const int tile = blockIdx.y * gridDim.x + blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m = st[ST_JM];
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  const double sref = coupling_ref(st), dcut = coupling_cut(st);
  // S is symmetric: tiles below the diagonal are written by their mirror
  if (i0 >= m || j0 >= m || conv || j0 < i0) {
    if (t == 0) aux[tile] = 0.0;
    return;
  }
  const int nch = (m + 15) / 16, nrb = nch;
  double av[DG_CH][4], bv[DG_CH][4];
#pragma unroll
  for (int u = 0; u < DG_CH; ++u) {
    const int c = wave + 4 * u;
    if (c < nch) {
      const int kb = 16 * c + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[u][q] = W[(size_t)(kb + q) * ld + i0 + r];
        bv[u][q] = T[(size_t)(kb + q) * ld + j0 + r];
      }
    }
  }
  // diagonal entries of the tile's rows and columns (lane r: row i0 + r and column j0 + r)
  double di = 0.0, dj = 0.0;
  if (wave == 0) {
    for (int b = 0; b < nrb; ++b) {
      di += Dp[(size_t)b * ld + i0 + r];
      dj += Dp[(size_t)b * ld + j0 + r];
    }
  }
  v4d acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int u = 0; u < DG_CH; ++u) {
    const int c = wave + 4 * u;
    if (c < nch) {
      const int kb = 16 * c + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = kb + q < m;
        const double a = keep_if(av[u][q], in), bb = keep_if(bv[u][q], in);
        if (q & 1) acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc2, 0, 0, 0);
        else acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc, 0, 0, 0);
      }
    }
  }
  acc += acc2;
  __shared__ double red[3][4][64];
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave > 0) return;
  double cmax = 0.0;
  const int j = j0 + r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = i0 + g + 4 * e;
    const double dii = __shfl(di, g + 4 * e, 64);
    if (i < m && j < m && j >= i) {
      const double o = acc[e] + red[0][e][lane] + red[1][e][lane] + red[2][e][lane];
      S[(size_t)i * ld + j] = o;
      S[(size_t)j * ld + i] = o;  // the mirror (the same value: S exactly symmetric)
      if (j > i) {
        const double c = coupling_at(o, dii, dj, sref, dcut);
        cmax = fmax(cmax, c);
        if (c > tol && fabs(o) > PCJ_OMEGA * fabs(dj - dii)) {
          const int slot = atomicAdd(&st[ST_NEDGE], 1);
          if (slot < EMAX) { edges[2 * slot] = i; edges[2 * slot + 1] = j; }
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o, 64));
  if (lane == 0) aux[tile] = cmax;
}

// ----------------------------------------------------------------------------
// Large-tile forms of the three fp64 GEMM kernels above, for batched launches
// over many paths: one workgroup per 96 x 96 output tile (9 per path at
// m <= 288) instead of one per 16 x 16 tile, so each operand panel is read
// from L2 six times less often. The depth is staged through LDS in chunks of
// 16 (double-buffered, one barrier per chunk; the next chunk's global loads
// are in flight during the current chunk's MFMAs). Wave (wr, wc) of the 2 x 2
// arrangement owns the 3 x 3 block of 16 x 16 sub-tiles at rows 48 wr and
// columns 48 wc; its MFMA operands come from LDS laid out k-major (As[k][i],
// Bs[k][j]) with a row stride of 112 doubles, so the two 16-lane halves of a
// fragment read fall on opposite halves of the banks. Depth entries >= m are
// zeroed as they enter LDS. Outputs, skip modes, diagonal partial sums and
// coupling maxima are those of the 16 x 16 kernels, with the same layouts.
constexpr int BT = 96;          // output tile edge
constexpr int BT_LD = 112;      // LDS row stride (doubles)
constexpr int BT_CH = 16 * BT_LD;  // doubles of one operand chunk in LDS

// Global -> registers for one depth chunk of one operand whose LDS form is
// X[k][x] = op(M)[x][k] (x in the tile's 96 indices). Transposed in memory
// (TM: M[k][x] row-major) the 16 rows of 96 are read along x; otherwise
// M[x][k] rows are read along k (16 values per row).
template <bool TM>
__device__ __forceinline__ void bt_load(const double* __restrict__ M, int ld, int x0, int k0, int t, double2 (&r)[3]) {
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int e = t + 256 * u;
    if (TM) {
      const int kk = e / 48, x2 = e % 48;
      r[u] = *(const double2*)(M + (size_t)(k0 + kk) * ld + x0 + 2 * x2);
    } else {
      const int x = e / 8, kk2 = e % 8;
      r[u] = *(const double2*)(M + (size_t)(x0 + x) * ld + k0 + 2 * kk2);
    }
  }
}

template <bool TM>
__device__ __forceinline__ void bt_store(double* X, int k0, int m, int t, const double2 (&r)[3]) {
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int e = t + 256 * u;
    if (TM) {
      const int kk = e / 48, x2 = e % 48;
      const bool in = k0 + kk < m;
      X[kk * BT_LD + 2 * x2] = keep_if(r[u].x, in);
      X[kk * BT_LD + 2 * x2 + 1] = keep_if(r[u].y, in);
    } else {
      const int x = e / 8, kk2 = e % 8;
      X[(2 * kk2) * BT_LD + x] = keep_if(r[u].x, k0 + 2 * kk2 < m);
      X[(2 * kk2 + 1) * BT_LD + x] = keep_if(r[u].y, k0 + 2 * kk2 + 1 < m);
    }
  }
}

// 4 k-steps of one chunk: acc[a][b] += As[:, 48 wr + 16 a] Bs[:, 48 wc + 16 b]
__device__ __forceinline__ void bt_mma(const double* As, const double* Bs, int wr, int wc, int lane,
                                       v4d (&acc)[3][3]) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = 4 * q + g;
    double af[3], bf[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) af[a] = As[k * BT_LD + 48 * wr + 16 * a + r];
#pragma unroll
    for (int b = 0; b < 3; ++b) bf[b] = Bs[k * BT_LD + 48 * wc + 16 * b + r];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int b = 0; b < 3; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[a], bf[b], acc[a][b], 0, 0, 0);
  }
}

// Main loop over the depth for one (DUAL: two) left operand(s) and one right
// operand; lds holds 2 buffers of (1 + DUAL) A chunks and one B chunk.
template <bool TA1, bool TA2, bool TB, bool DUAL>
__device__ __forceinline__ void bt_mainloop(const double* A1, const double* A2, const double* B, int ld, int m,
                                            int i0, int j0, double* lds, v4d (&acc1)[3][3], v4d (&acc2)[3][3]) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  constexpr int NB = DUAL ? 3 : 2;  // chunks per buffer
  const int nch = (m + 15) / 16;
  double2 ra1[3], ra2[3], rb[3];
  bt_load<TA1>(A1, ld, i0, 0, t, ra1);
  if (DUAL) bt_load<TA2>(A2, ld, i0, 0, t, ra2);
  bt_load<!TB>(B, ld, j0, 0, t, rb);
  for (int c = 0; c < nch; ++c) {
    double* buf = lds + (c & 1) * NB * BT_CH;
    bt_store<TA1>(buf, 16 * c, m, t, ra1);
    if (DUAL) bt_store<TA2>(buf + 2 * BT_CH, 16 * c, m, t, ra2);
    bt_store<!TB>(buf + BT_CH, 16 * c, m, t, rb);
    __syncthreads();
    if (c + 1 < nch) {
      bt_load<TA1>(A1, ld, i0, 16 * (c + 1), t, ra1);
      if (DUAL) bt_load<TA2>(A2, ld, i0, 16 * (c + 1), t, ra2);
      bt_load<!TB>(B, ld, j0, 16 * (c + 1), t, rb);
    }
    bt_mma(buf, buf + BT_CH, wr, wc, lane, acc1);
    if (DUAL) bt_mma(buf + 2 * BT_CH, buf + BT_CH, wr, wc, lane, acc2);
  }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void bgemm_kernel(const double* __restrict__ A, const double* __restrict__ B,
                                                    double* C, const double* Cin, int ld, double alpha, double beta,
                                                    double gamma, const int32_t* __restrict__ st, int mode,
                                                    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A = iskv_rb(A, bdel);
  B = iskv_rb(B, bdel);
  C = iskv_rb(C, bdel);
  Cin = iskv_rb(Cin, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * BT, j0 = blockIdx.x * BT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int m = st[ST_JM];
  if (i0 >= m || j0 >= m) return;
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  if ((mode == 0 || mode == 3) && conv) return;
  if (mode == 1 && conv) {
    for (int e = t; e < BT * BT; e += 256) {
      const int i = i0 + e / BT, j = j0 + e % BT;
      if (i < m && j < m) C[(size_t)i * ld + j] = Cin[(size_t)i * ld + j];
    }
    return;
  }
  extern __shared__ double bt_lds[];
  v4d acc[3][3], unused[3][3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) acc[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
  bt_mainloop<TA, false, TB, false>(A, nullptr, B, ld, m, i0, j0, bt_lds, acc, unused);
  const int r = lane & 15, g = lane >> 4, wr = wave >> 1, wc = wave & 1;
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 48 * wr + 16 * a + g + 4 * e, j = j0 + 48 * wc + 16 * b + r;
        if (i < m && j < m) {
          double o = alpha * acc[a][b][e];
          if (beta != 0.0) o += beta * Cin[(size_t)i * ld + j];
          if (i == j) o += gamma;
          C[(size_t)i * ld + j] = o;
        }
      }
}

template <bool TA1, bool TA2>
__global__ __launch_bounds__(256) void bgemm2_kernel(const double* __restrict__ A1, const double* __restrict__ A2,
                                                     const double* __restrict__ B, int ld, double* C1, double* C2,
                                                     const double* Cin1, const double* Cin2, double alpha1,
                                                     double beta1, double alpha2, double beta2, double* Dp,
                                                     const int32_t* __restrict__ st, int mode,
                                                     const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A1 = iskv_rb(A1, bdel);
  A2 = iskv_rb(A2, bdel);
  B = iskv_rb(B, bdel);
  C1 = iskv_rb(C1, bdel);
  C2 = iskv_rb(C2, bdel);
  Cin1 = iskv_rb(Cin1, bdel);
  Cin2 = iskv_rb(Cin2, bdel);
  Dp = iskv_rb(Dp, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * BT, j0 = blockIdx.x * BT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int m = st[ST_JM];
  if (i0 >= m || j0 >= m) return;
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  if (mode == 0 && conv) return;
  if (mode == 4 && conv && st[ST_PCJIT] > 0 && !(st[ST_PCJ] & FLAG_NS)) return;
  if (mode == 1 && conv) {
    for (int e = t; e < BT * BT; e += 256) {
      const int i = i0 + e / BT, j = j0 + e % BT;
      if (i < m && j < m) {
        C1[(size_t)i * ld + j] = Cin1[(size_t)i * ld + j];
        C2[(size_t)i * ld + j] = Cin2[(size_t)i * ld + j];
      }
    }
    return;
  }
  extern __shared__ double bt_lds[];
  v4d acc1[3][3], acc2[3][3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) acc1[a][b] = acc2[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
  bt_mainloop<TA1, TA2, false, true>(A1, A2, B, ld, m, i0, j0, bt_lds, acc1, acc2);
  const int r = lane & 15, g = lane >> 4, wr = wave >> 1, wc = wave & 1;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int ib = i0 + 48 * wr + 16 * a;  // first row of the sub-tile
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int j = j0 + 48 * wc + 16 * b + r;
      double dsum = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ib + g + 4 * e;
        if (i < m && j < m) {
          double o1 = alpha1 * acc1[a][b][e], o2 = alpha2 * acc2[a][b][e];
          if (beta1 != 0.0) o1 += beta1 * Cin1[(size_t)i * ld + j];
          if (beta2 != 0.0) o2 += beta2 * Cin2[(size_t)i * ld + j];
          C1[(size_t)i * ld + j] = o1;
          C2[(size_t)i * ld + j] = o2;
          dsum = fma(o1, o2, dsum);
        }
      }
      if (Dp) {
        dsum += __shfl_xor(dsum, 16, 64);
        dsum += __shfl_xor(dsum, 32, 64);
        if (g == 0 && ib < m) Dp[(size_t)(ib / 16) * ld + j] = dsum;
      }
    }
  }
}

// S = W^T T with the strong-pair detection (as dgemm_s_kernel); the coupling
// maximum of 16 x 16 sub-tile (I, J) goes to aux[I nblk + J].
__global__ __launch_bounds__(256) void bgemm_s_kernel(const double* __restrict__ W, const double* __restrict__ T,
                                                      int ld, double* S, const double* __restrict__ Dp,
                                                      double* aux, int nblk, int* edges, int32_t* st, double tol,
                                                      const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  W = iskv_rb(W, bdel);
  T = iskv_rb(T, bdel);
  S = iskv_rb(S, bdel);
  Dp = iskv_rb(Dp, bdel);
  aux = iskv_rb(aux, bdel);
  edges = iskv_rb(edges, bdel);
  st = iskv_rb(st, bdel);
  const int i0 = blockIdx.y * BT, j0 = blockIdx.x * BT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, g = lane >> 4, wr = wave >> 1, wc = wave & 1;
  const int m = st[ST_JM];
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  const double sref = coupling_ref(st), dcut = coupling_cut(st);
  // S is symmetric: tiles below the diagonal are written by their mirror
  if (i0 >= m || j0 >= m || conv || j0 < i0) {
    // every sub-tile maximum of this tile is 0
    if (t < 36) {
      const int I = i0 / 16 + t / 6, J = j0 / 16 + t % 6;
      if (I < nblk && J < nblk) aux[I * nblk + J] = 0.0;
    }
    return;
  }
  extern __shared__ double bt_lds[];
  v4d acc[3][3], unused[3][3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) acc[a][b] = v4d{0.0, 0.0, 0.0, 0.0};
  bt_mainloop<true, false, false, false>(W, nullptr, T, ld, m, i0, j0, bt_lds, acc, unused);
  const int nrb = (m + 15) / 16;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int ib = i0 + 48 * wr + 16 * a;
    double di = 0.0;
    for (int b2 = 0; b2 < nrb; ++b2) di += Dp[(size_t)b2 * ld + ib + r];
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      const int jb = j0 + 48 * wc + 16 * b, j = jb + r;
      double dj = 0.0;
      for (int b2 = 0; b2 < nrb; ++b2) dj += Dp[(size_t)b2 * ld + j];
      double cmax = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = ib + g + 4 * e;
        const double dii = __shfl(di, g + 4 * e, 64);
        if (i < m && j < m && j >= i) {
          const double o = acc[a][b][e];
          S[(size_t)i * ld + j] = o;
          S[(size_t)j * ld + i] = o;
          if (j > i) {
            const double c = coupling_at(o, dii, dj, sref, dcut);
            cmax = fmax(cmax, c);
            if (c > tol && fabs(o) > PCJ_OMEGA * fabs(dj - dii)) {
              const int slot = atomicAdd(&st[ST_NEDGE], 1);
              if (slot < EMAX) { edges[2 * slot] = i; edges[2 * slot + 1] = j; }
            }
          }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o, 64));
      if (lane == 0 && ib / 16 < nblk && jb / 16 < nblk) aux[(ib / 16) * nblk + jb / 16] = cmax;
    }
  }
}

static inline size_t bt_lds_bytes(bool dual) { return (size_t)2 * (dual ? 3 : 2) * BT_CH * sizeof(double); }

// Batched launches over at least this many paths use the 96 x 96 tiles.
constexpr int BT_MIN_BATCH = 16;

// C = alpha op(A) op(B) + beta Cin + gamma I, tile size chosen by batch size.
template <bool TA, bool TB>
void gemm(hipStream_t s, int m_max, const double* A, const double* B, double* C, const double* Cin, int ld,
          double alpha, double beta, double gamma, const int32_t* st, int mode, const int64_t* bd, int bc) {
  if (bc >= BT_MIN_BATCH) {
    const int nt = (m_max + BT - 1) / BT;
    hipLaunchKernelGGL((bgemm_kernel<TA, TB>), bz(dim3(nt, nt), bc), dim3(256), bt_lds_bytes(false), s, A, B, C,
                       Cin, ld, alpha, beta, gamma, st, mode, bd);
  } else {
    dgemm<TA, TB>(s, m_max, A, B, C, Cin, ld, alpha, beta, gamma, st, mode, bd, bc);
  }
}

// C1 = alpha1 op(A1) B + beta1 Cin1, C2 = alpha2 op(A2) B + beta2 Cin2 (+ Dp).
template <bool TA1, bool TA2>
void gemm2(hipStream_t s, int m_max, const double* A1, const double* A2, const double* B, int ld, double* C1,
           double* C2, const double* Cin1, const double* Cin2, double alpha1, double beta1, double alpha2,
           double beta2, double* Dp, const int32_t* st, int mode, const int64_t* bd, int bc) {
  if (bc >= BT_MIN_BATCH) {
    const int nt = (m_max + BT - 1) / BT;
    hipLaunchKernelGGL((bgemm2_kernel<TA1, TA2>), bz(dim3(nt, nt), bc), dim3(256), bt_lds_bytes(true), s, A1, A2,
                       B, ld, C1, C2, Cin1, Cin2, alpha1, beta1, alpha2, beta2, Dp, st, mode, bd);
  } else {
    const int nb = (m_max + 15) / 16;
    hipLaunchKernelGGL((dgemm2_kernel<TA1, TA2, DG2_NW>), bz(dim3(nb, nb), bc), dim3(64 * DG2_NW), 0, s, A1, A2, B,
                       ld, C1, C2,
                       Cin1, Cin2, alpha1, beta1, alpha2, beta2, Dp, st, mode, bd);
  }
}

// S = W^T T with strong-pair detection (aux: nblk x nblk maxima).
void gemm_s(hipStream_t s, int m_max, const double* W, const double* T, int ld, double* S, const double* Dp,
            double* aux, int* edges, int32_t* st, double tol, const int64_t* bd, int bc) {
  const int nb = (m_max + 15) / 16;
  if (bc >= BT_MIN_BATCH) {
    const int nt = (m_max + BT - 1) / BT;
    hipLaunchKernelGGL(bgemm_s_kernel, bz(dim3(nt, nt), bc), dim3(256), bt_lds_bytes(false), s, W, T, ld, S, Dp,
                       aux, nb, edges, st, tol, bd);
  } else {
    hipLaunchKernelGGL(dgemm_s_kernel, bz(dim3(nb, nb), bc), dim3(256), 0, s, W, T, ld, S, Dp, aux, edges, st, tol,
                       bd);
  }
}

// S = A, W = I, flags cleared.
__global__ __launch_bounds__(256) void pcj_init_kernel(const double* __restrict__ A, double* S,
                                                       double* W, int ld, int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A = iskv_rb(A, bdel);
  S = iskv_rb(S, bdel);
  W = iskv_rb(W, bdel);
  st = iskv_rb(st, bdel);
  const int m = st[ST_JM];
  const size_t total = (size_t)m * m;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / m), j = (int)(e % m);
    S[(size_t)i * ld + j] = A[(size_t)i * ld + j];
    W[(size_t)i * ld + j] = (i == j) ? 1.0 : 0.0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) { st[ST_PCJ] = 0; st[ST_PCJIT] = 0; st[ST_NEDGE] = 0; st[ST_ROUNDS] = 0; }
}


__device__ __forceinline__ void rot2(double app, double aqq, double apq, double* c, double* s) {
  double tau = (aqq - app) / (2.0 * apq);
  double tt = (tau >= 0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
  *c = 1.0 / sqrt(1.0 + tt * tt);
  *s = tt * (*c);
}

// Cyclic Jacobi on a c x c cluster block (c <= CMAX_S) by a group of 8 lanes
// of one wave: lane x < c holds row x of the block (srow) and of the
// eigenvector matrix (vrow) in registers. Every lane of the group forms the
// same rotation from values shuffled out of lanes p and q; the column update
// is local, the row update exchanges rows p and q. `base` is the group's
// first lane in the wave. Sweeps end when one rotates nothing (the decision
// is the same in every lane of the group).
// One rotation (p, q) of jacobi_group, with compile-time indices so the
// row arrays stay in registers.
template <int P, int Q>
__device__ __forceinline__ void jacobi_pair(double (&srow)[CMAX_S], double (&vrow)[CMAX_S], int c, int x, int base,
                                            bool& rotated) {
  if (Q >= c) return;
  const double app = __shfl(srow[P], base + P, 64);
  const double aqq = __shfl(srow[Q], base + Q, 64);
  const double apq = __shfl(srow[Q], base + P, 64);
  if (apq == 0.0 || !(fabs(apq) > 1e-14 * sqrt(fabs(app * aqq)))) return;
  double cs, sn;
  rot2(app, aqq, apq, &cs, &sn);
  rotated = true;
  {  // columns P, Q of the block and of V
    const double sp = srow[P], sq = srow[Q];
    srow[P] = cs * sp - sn * sq;
    srow[Q] = sn * sp + cs * sq;
    const double vp = vrow[P], vq = vrow[Q];
    vrow[P] = cs * vp - sn * vq;
    vrow[Q] = sn * vp + cs * vq;
  }
  const int partner = base + (x == P ? Q : P);
#pragma unroll
  for (int y = 0; y < CMAX_S; ++y) {  // rows P, Q
    const double o = __shfl(srow[y], partner, 64);
    if (x == P) srow[y] = cs * srow[y] - sn * o;
    else if (x == Q) srow[y] = sn * o + cs * srow[y];
  }
}

template <int P, int Q>
__device__ __forceinline__ void jacobi_sweep(double (&srow)[CMAX_S], double (&vrow)[CMAX_S], int c, int x, int base,
                                             bool& rotated) {
  if constexpr (P < CMAX_S - 1) {
    jacobi_pair<P, Q>(srow, vrow, c, x, base, rotated);
    if constexpr (Q + 1 < CMAX_S) jacobi_sweep<P, Q + 1>(srow, vrow, c, x, base, rotated);
    else jacobi_sweep<P + 1, P + 2>(srow, vrow, c, x, base, rotated);
  }
}

__device__ void jacobi_group(double (&srow)[CMAX_S], double (&vrow)[CMAX_S], int c, int x, int base) {
  for (int sweep = 0; sweep < 20; ++sweep) {
    bool rotated = false;
    jacobi_sweep<0, 1>(srow, vrow, c, x, base, rotated);
    if (!rotated) break;
  }
}

// Strong pairs and per-tile maxima of the scaled coupling, one 16 x 16 tile
// of S per workgroup (first refinement step, where S = A; later steps detect
// in the epilogue of the GEMM that forms S). Tile (bi, bj) with bj >= bi
// checks its pairs i < j and writes its largest coupling to aux[bi nb + bj]
// (tiles below the diagonal write 0). Strong pairs are appended to the edge
// list (order fixed later by sorting). Each entry's load is issued before the
// coupling scale and cut are formed, so the two latencies overlap.
__global__ __launch_bounds__(256) void pcj_detect_kernel(const double* __restrict__ S, int ld,
                                                         double* aux, int* edges, int32_t* st, double tol, int keep,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  aux = iskv_rb(aux, bdel);
  edges = iskv_rb(edges, bdel);
  st = iskv_rb(st, bdel);
  if (st[ST_PCJ] & FLAG_CONV) return;
  const int m = st[ST_JM];
  const int bi = blockIdx.y, bj = blockIdx.x, tile = bi * gridDim.x + bj;
  const int i = 16 * bi + (threadIdx.x >> 4), j = 16 * bj + (threadIdx.x & 15);
  if (bj < bi || 16 * bi >= m || 16 * bj >= m) {
    if (threadIdx.x == 0) aux[tile] = 0.0;
    return;
  }
  const bool pair = i < m && j < m && j > i;
  const double sij = pair ? S[(size_t)i * ld + j] : 0.0;
  __shared__ double red[4];
  // coupling scale (the largest diagonal entry) and cut (between the keep-th
  // and (keep+1)-th largest diagonal entries, geometric mean), rounded to
  // fp32 so that the later steps (reading them from st) use the same values;
  // every workgroup forms them from S = A, tile (0, 0) publishes them.
  // keep < 0: scaled couplings; keep >= m: nothing dropped.
  __shared__ double dg[1024], dl[1024];
  __shared__ double cred[3][4];
  double dmax = 0.0, hi = INFINITY, lo = 0.0;
  for (int e = threadIdx.x; e < m; e += 256) {
    const double d = S[(size_t)e * ld + e];
    dg[e] = d;
    dl[e] = fabs(d);
    dmax = fmax(dmax, fabs(d));
  }
  __syncthreads();
  if (keep >= 0 && keep < m)
    for (int e = threadIdx.x; e < m; e += 256) {
      const double v = dl[e];
      int above = 0;
#pragma unroll 8
      for (int q = 0; q < m; ++q) above += dl[q] > v;
      if (above < keep) hi = fmin(hi, v);
      else lo = fmax(lo, v);
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    dmax = fmax(dmax, __shfl_xor(dmax, o, 64));
    hi = fmin(hi, __shfl_xor(hi, o, 64));
    lo = fmax(lo, __shfl_xor(lo, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    cred[0][threadIdx.x >> 6] = dmax;
    cred[1][threadIdx.x >> 6] = hi;
    cred[2][threadIdx.x >> 6] = lo;
  }
  __syncthreads();
  dmax = fmax(fmax(cred[0][0], cred[0][1]), fmax(cred[0][2], cred[0][3]));
  hi = fmin(fmin(cred[1][0], cred[1][1]), fmin(cred[1][2], cred[1][3]));
  lo = fmax(fmax(cred[2][0], cred[2][1]), fmax(cred[2][2], cred[2][3]));
  auto up = [](double x) {
    const float f = (float)x;
    return (double)f < x ? __int_as_float(__float_as_int(f) + 1) : f;
  };
  const float fu = up(dmax);
  const bool prod = keep >= 0 && isfinite(fu) && fu > 0.f;
  const double cut = (keep >= 0 && keep < m && isfinite(hi)) ? sqrt(hi * lo) : -1.0;
  const float fcut = prod && cut >= 0.0 ? (float)cut : -1.f;
  const double sref = prod ? (double)fu : 0.0, dcut = (double)fcut;
  if (tile == 0 && threadIdx.x == 0) {
    st[ST_SREF] = prod ? __float_as_int(fu) : 0;
    st[ST_DCUT] = __float_as_int(fcut);
  }
  double cmax = 0.0;
  if (pair) {
    const double di = dg[i], dj = dg[j];
    const double c = coupling_at(sij, di, dj, sref, dcut);
    cmax = c;
    if (c > tol && fabs(sij) > PCJ_OMEGA * fabs(dj - di)) {
      int slot = atomicAdd(&st[ST_NEDGE], 1);
      if (slot < EMAX) { edges[2 * slot] = i; edges[2 * slot + 1] = j; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cmax;
  __syncthreads();
  if (threadIdx.x == 0) aux[tile] = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
}

struct AnalyzeLds {
  double d[1024];
  int key[EMAX];
  int lab[1024];
  int size[1024];
  int cid[1024];
  int members[NCL_MAX][CMAX_S];
  int ccount[NCL_MAX];
  int pi[NPAIR_MAX], pj[NPAIR_MAX];
  unsigned char used[1024];
  double cmax;
  int nedge, ncl, npair, changed, anybig;
};

// The serial part of one refinement step, one workgroup of 1024 threads:
// convergence test, clusters of strongly coupled indices (components of the
// strong-pair graph), exact rotations (small clusters: cyclic Jacobi; big
// ones: 2x2 rotations on a greedy matching), published as rotation tables
// that the angle kernel applies to S (on the fly) and W.
__global__ __launch_bounds__(1024) void pcj_analyze_kernel(const double* __restrict__ S, int ld,
                                                           const double* __restrict__ aux, int nmx,
                                                           const int* __restrict__ edges, int32_t* itab,
                                                           double* rtab, int mmax, int32_t* st, int it, double tol,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  aux = iskv_rb(aux, bdel);
  edges = iskv_rb(edges, bdel);
  itab = iskv_rb(itab, bdel);
  rtab = iskv_rb(rtab, bdel);
  st = iskv_rb(st, bdel);
  extern __shared__ unsigned char smem_raw[];
  AnalyzeLds& L = *reinterpret_cast<AnalyzeLds*>(smem_raw);
  if (st[ST_PCJ] & FLAG_CONV) return;
  const int m = st[ST_JM];
  const int t = threadIdx.x, nt = blockDim.x;
  if (t < 64) {
    double c = 0.0;
    for (int b = t; b < nmx; b += 64) c = fmax(c, aux[b]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c = fmax(c, __shfl_xor(c, o, 64));
    if (t == 0) {
      L.cmax = c;
      int ne = st[ST_NEDGE];
      L.nedge = ne < EMAX ? ne : EMAX;
      L.ncl = 0; L.npair = 0; L.anybig = 0;
    }
  }
  __syncthreads();
  const double cmax = L.cmax;
  if (cmax < tol) {  // NaN couplings never pass: they end in the fallback
    __syncthreads();
    if (t == 0) { st[ST_PCJ] |= FLAG_CONV; st[ST_PCJIT] = it; st[ST_NEDGE] = 0; }
    return;
  }
  const int ne = L.nedge;
  for (int i = t; i < m; i += nt) L.d[i] = S[(size_t)i * ld + i];
  if (ne == 0) {  // no strongly coupled pair: the first-order angles do everything
    if (t == 0) { st[ST_NEDGE] = 0; st[ST_PCJIT] = it + 1; st[ST_NROT] = 0; }
    return;
  }
  for (int e = t; e < ne; e += nt) L.key[e] = edges[2 * e] * 1024 + edges[2 * e + 1];
  for (int i = t; i < m; i += nt) { L.lab[i] = i; L.size[i] = 0; L.used[i] = 0; L.cid[i] = -1; }
  __syncthreads();
  // connected components by min-label propagation
  for (int guard = 0; guard < 1024; ++guard) {
    if (t == 0) L.changed = 0;
    __syncthreads();
    for (int e = t; e < ne; e += nt) {
      int a = L.key[e] >> 10, b = L.key[e] & 1023;
      int la = L.lab[a], lb = L.lab[b];
      if (la != lb) {
        int l = la < lb ? la : lb;
        atomicMin(&L.lab[a], l);
        atomicMin(&L.lab[b], l);
        L.changed = 1;
      }
    }
    __syncthreads();
    for (int i = t; i < m; i += nt) L.lab[i] = L.lab[L.lab[i]];  // pointer jumping
    __syncthreads();
    // every thread reads the flag before thread 0 may reset it for the next
    // pass, so the loop exit is uniform across the workgroup
    const int ch = L.changed;
    __syncthreads();
    if (!ch) break;
  }
  for (int i = t; i < m; i += nt) atomicAdd(&L.size[L.lab[i]], 1);
  __syncthreads();
  // small clusters (2..CMAX_S) get ids in root order (prefix count over
  // roots); larger components are "big"
  if (t < 64) {
    int base = 0;
    for (int i0 = 0; i0 < m; i0 += 64) {
      int i = i0 + t;
      bool small = i < m && L.lab[i] == i && L.size[i] >= 2 && L.size[i] <= CMAX_S;
      bool big = i < m && L.lab[i] == i && L.size[i] > CMAX_S;
      unsigned long long ms = __ballot(small);
      if (__ballot(big)) L.anybig = 1;
      int id = base + __popcll(ms & ((1ull << t) - 1ull));
      if (small) {
        if (id < NCL_MAX) { L.cid[i] = id; L.ccount[id] = 0; }
        else L.anybig = 1;
      }
      base += __popcll(ms);
    }
    if (t == 0) L.ncl = base < NCL_MAX ? base : NCL_MAX;
  }
  __syncthreads();
  for (int i = t; i < m; i += nt) {
    int c = L.cid[L.lab[i]];
    if (c >= 0) L.members[c][atomicAdd(&L.ccount[c], 1)] = i;
  }
  __syncthreads();
  if (t < L.ncl) {  // members in index order (deterministic)
    const int c = L.ccount[t];
    for (int a = 1; a < c; ++a) {
      int v = L.members[t][a], b2 = a - 1;
      while (b2 >= 0 && L.members[t][b2] > v) { L.members[t][b2 + 1] = L.members[t][b2]; --b2; }
      L.members[t][b2 + 1] = v;
    }
  }
  if (L.anybig) {
    // greedy matching on strong pairs inside big components, in sorted pair
    // order so the result does not depend on the detection order
    int npow = 1;
    while (npow < ne) npow <<= 1;
    for (int e = ne + t; e < npow; e += nt) L.key[e] = 0x7fffffff;
    __syncthreads();
    for (int k = 2; k <= npow; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int e = t; e < npow; e += nt) {
          int p = e ^ j;
          if (p > e) {
            int a = L.key[e], b = L.key[p];
            bool up = (e & k) == 0;
            if ((a > b) == up) { L.key[e] = b; L.key[p] = a; }
          }
        }
        __syncthreads();
      }
    }
    if (t == 0) {
      int np = 0;
      for (int e = 0; e < ne && np < NPAIR_MAX; ++e) {
        int a = L.key[e] >> 10, b = L.key[e] & 1023;
        if (L.cid[L.lab[a]] >= 0) continue;
        if (L.used[a] || L.used[b]) continue;
        L.used[a] = 1; L.used[b] = 1;
        L.pi[np] = a; L.pj[np] = b;
        ++np;
      }
      L.npair = np;
    }
  }
  if (t == 0) st[ST_NEDGE] = 0;  // the next detect pass starts a new list
  __syncthreads();
  const int ncl = L.ncl, npair = L.npair;
  // the step's exact rotations go to the tables that the angle kernel
  // applies: group of each index (or -1) and its place, group sizes and
  // members, the rotated diagonal of the members, each group's rotation R
  // (columns = the rotated directions, W <- W R)
  int32_t* gid = itab;
  int32_t* gpos = itab + mmax;
  int32_t* gcnt = itab + 2 * mmax;
  int32_t* gmem = gcnt + (mmax / 2 + 1);
  double* drot = rtab;
  double* Rg = rtab + mmax;
  for (int i = t; i < m; i += nt) gid[i] = -1;
  __syncthreads();
  if ((t >> 3) < ncl) {  // cluster t / 8 on lanes 8 (t / 8) .. +7
    const int g = t >> 3, x = t & 7, c = L.ccount[g];
    double srow[CMAX_S], vrow[CMAX_S];
#pragma unroll
    for (int b = 0; b < CMAX_S; ++b) {
      srow[b] = (x < c && b < c) ? S[(size_t)L.members[g][x] * ld + L.members[g][b]] : 0.0;
      vrow[b] = (x == b) ? 1.0 : 0.0;
    }
    jacobi_group(srow, vrow, c, x, (t & 63) & ~7);
    if (x < c) {
      const int mx = L.members[g][x];
      gid[mx] = g;
      gpos[mx] = x;
      gmem[g * CMAX_S + x] = mx;
#pragma unroll
      for (int b = 0; b < CMAX_S; ++b) {
        if (b < c) Rg[(size_t)g * CMAX_S * CMAX_S + x * CMAX_S + b] = vrow[b];
        if (b == x) drot[mx] = srow[b];
      }
      if (x == 0) gcnt[g] = c;
    }
  }
  for (int q = t; q < npair; q += nt) {
    const int a = L.pi[q], b = L.pj[q], g = ncl + q;
    double cs = 1.0, sn = 0.0;
    const double apq = S[(size_t)a * ld + b], da = L.d[a], db = L.d[b];
    if (apq != 0.0) rot2(da, db, apq, &cs, &sn);
    gid[a] = g; gpos[a] = 0; gid[b] = g; gpos[b] = 1;
    gcnt[g] = 2;
    gmem[g * CMAX_S] = a;
    gmem[g * CMAX_S + 1] = b;
    double* R = Rg + (size_t)g * CMAX_S * CMAX_S;  // [[c, s], [-s, c]]
    R[0] = cs; R[1] = sn; R[CMAX_S] = -sn; R[CMAX_S + 1] = cs;
    drot[a] = cs * cs * da - 2.0 * cs * sn * apq + sn * sn * db;
    drot[b] = sn * sn * da + 2.0 * cs * sn * apq + cs * cs * db;
  }
  if (t == 0) { st[ST_PCJIT] = it + 1; st[ST_NROT] = ncl + npair; }
}

// First-order angles for every pair that is not strongly coupled, from
// S' = R^T S R, S rotated by the step's exact rotations R (block diagonal
// over the analysis' rotation groups, identity elsewhere): K_ij =
// s'_ij / (s'_jj - s'_ii), K antisymmetric, clipped; writes Km = K and
// Pa = I + K/2 (X = I + K (I + K/2) is formed by one GEMM). An entry of S'
// is formed from the groups of its row and column (pairs inside one group
// are diagonalised: zero). The same launch applies R to W: W[:, g] <- W[:, g] R_g
// for every group g (rows and groups disjoint, in place). Grid-stride, many
// workgroups.
__global__ __launch_bounds__(256) void pcj_kmat_kernel(const double* __restrict__ S, int ld, double* Km,
                                                       double* Pa, double* W, const int32_t* __restrict__ itab,
                                                       const double* __restrict__ rtab, int mmax,
                                                       const int32_t* __restrict__ st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  Km = iskv_rb(Km, bdel);
  Pa = iskv_rb(Pa, bdel);
  W = iskv_rb(W, bdel);
  itab = iskv_rb(itab, bdel);
  rtab = iskv_rb(rtab, bdel);
  st = iskv_rb(st, bdel);
  if (st[ST_PCJ] & FLAG_CONV) return;
  const int m = st[ST_JM];
  const int nrot = st[ST_NROT];
  const int32_t* gid = itab;
  const int32_t* gpos = itab + mmax;
  const int32_t* gcnt = itab + 2 * mmax;
  const int32_t* gmem = gcnt + (mmax / 2 + 1);
  const double* drot = rtab;
  const double* Rg = rtab + mmax;
  const size_t tot = (size_t)m * m;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += stride) {
    int i = (int)(e / m), j = (int)(e % m);
    double k = 0.0;
    if (i != j) {
      int lo = i < j ? i : j, hi = i < j ? j : i;
      const int gl = nrot > 0 ? gid[lo] : -1, gh = nrot > 0 ? gid[hi] : -1;
      double slh, dl, dh;
      if (gl < 0 && gh < 0) {
        slh = S[(size_t)lo * ld + hi];
        dl = S[(size_t)lo * ld + lo];
        dh = S[(size_t)hi * ld + hi];
      } else {
        dl = gl >= 0 ? drot[lo] : S[(size_t)lo * ld + lo];
        dh = gh >= 0 ? drot[hi] : S[(size_t)hi * ld + hi];
        slh = 0.0;
        if (gl != gh) {
          const int cl = gl >= 0 ? gcnt[gl] : 1, ch = gh >= 0 ? gcnt[gh] : 1;
          const int pl = gl >= 0 ? gpos[lo] : 0, ph = gh >= 0 ? gpos[hi] : 0;
          for (int a = 0; a < cl; ++a) {
            const int ma = gl >= 0 ? gmem[gl * CMAX_S + a] : lo;
            const double ra = gl >= 0 ? Rg[(size_t)gl * CMAX_S * CMAX_S + a * CMAX_S + pl] : 1.0;
            double row = 0.0;
            for (int b = 0; b < ch; ++b) {
              const int mb = gh >= 0 ? gmem[gh * CMAX_S + b] : hi;
              const double rb = gh >= 0 ? Rg[(size_t)gh * CMAX_S * CMAX_S + b * CMAX_S + ph] : 1.0;
              row = fma(S[(size_t)ma * ld + mb], rb, row);
            }
            slh = fma(ra, row, slh);
          }
        }
      }
      const double den = dh - dl;
      if (den != 0.0 && fabs(slh) <= PCJ_OMEGA * fabs(den)) k = fmin(fmax(slh / den, -PCJ_CLIP), PCJ_CLIP);
      if (!isfinite(k)) k = 0.0;
      if (i > j) k = -k;
    }
    Km[(size_t)i * ld + j] = k;
    Pa[(size_t)i * ld + j] = (i == j ? 1.0 : 0.0) + 0.5 * k;
  }
  // W[i, members of g] <- W[i, members of g] R_g
  const size_t wtot = (size_t)m * nrot;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < wtot; e += stride) {
    const int i = (int)(e / nrot), g = (int)(e % nrot);
    const int c = gcnt[g];
    double w[CMAX_S];
#pragma unroll
    for (int a = 0; a < CMAX_S; ++a) w[a] = a < c ? W[(size_t)i * ld + gmem[g * CMAX_S + a]] : 0.0;
    const double* R = Rg + (size_t)g * CMAX_S * CMAX_S;
#pragma unroll
    for (int b = 0; b < CMAX_S; ++b) {
      if (b >= c) continue;
      double acc = 0.0;
#pragma unroll
      for (int a = 0; a < CMAX_S; ++a)
        if (a < c) acc = fma(w[a], R[a * CMAX_S + b], acc);
      W[(size_t)i * ld + gmem[g * CMAX_S + b]] = acc;
    }
  }
}

// A converged refinement also needs an orthonormal W: W^T A W diagonal does
// not imply it (inside a cluster of nearly equal eigenvalues the columns can
// drift towards each other while the couplings stay small). T = W^T W of the
// W before its final Newton-Schulz step: any |T - I| above thr withdraws the
// convergence and marks the fallback cold (ST_ROUNDS = 1). Without
// convergence the same test keeps the fallback from continuing from a W that
// is not orthonormal (cold instead of warm). Grid-stride.
__global__ __launch_bounds__(256) void pcj_orth_check_kernel(const double* __restrict__ T, int ld, int32_t* st,
                                                             double thr, int pre, const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  T = iskv_rb(T, bdel);
  st = iskv_rb(st, bdel);
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  // pre: after convergence at a step >= 1, T = W^T W of the iterate behind
  // the orthonormalised W; a defect above thr asks for the final step
  if (pre && !(conv && st[ST_PCJIT] > 0)) return;
  const int m = st[ST_JM];
  const size_t tot = (size_t)m * m;
  bool bad = false;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    const size_t i = e / m, j = e % m;
    const double v = T[i * ld + j] - (i == j ? 1.0 : 0.0);
    bad |= !(fabs(v) <= thr);
  }
  if (bad && pre) {
    atomicOr(&st[ST_PCJ], FLAG_NS);
  } else if (bad) {
    if (conv) atomicAnd(&st[ST_PCJ], ~FLAG_CONV);
    st[ST_ROUNDS] = 1;
  }
}

// Eigenvalues lambda_i = w_i^T (A w_i) from T = A W; V = W when converged.
// W is Wo, the last step's orthonormalised iterate, when the refinement
// converged at a step >= 1 (the final paired products were skipped), else Wf
// from the final Newton-Schulz step.
// Otherwise the Jacobi fallback takes over: when the last step's couplings
// (aux, nmx maxima) are all finite and below 0.05, it continues from
// S = Wf^T A Wf (formed by the launch before) and V = Wf, nearly diagonal so
// that a few sweeps finish it; else it starts from S = A, V = I (FLAG_COLD).
// Grid (m).
__global__ __launch_bounds__(256) void pcj_final_kernel(const double* __restrict__ Wo,
                                                        const double* __restrict__ Wf,
                                                        const double* __restrict__ T,
                                                        const double* __restrict__ A, double* S,
                                                        double* V, int ld, const double* __restrict__ aux,
                                                        int nmx, int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  Wo = iskv_rb(Wo, bdel);
  Wf = iskv_rb(Wf, bdel);
  aux = iskv_rb(aux, bdel);
  T = iskv_rb(T, bdel);
  A = iskv_rb(A, bdel);
  S = iskv_rb(S, bdel);
  V = iskv_rb(V, bdel);
  st = iskv_rb(st, bdel);
  const int m = st[ST_JM];
  const int j = blockIdx.x;
  if (j >= m) return;
  const bool conv = (st[ST_PCJ] & FLAG_CONV) != 0;
  __shared__ double red[4];
  if (conv) {
    const double* Wv = (st[ST_PCJIT] > 0 && !(st[ST_PCJ] & FLAG_NS)) ? Wo : Wf;
    double acc = 0.0;
    for (int r = threadIdx.x; r < m; r += 256) {
      double w = Wv[(size_t)r * ld + j];
      acc = fma(w, T[(size_t)r * ld + j], acc);
      V[(size_t)r * ld + j] = w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) S[(size_t)j * ld + j] = red[0] + red[1] + red[2] + red[3];
  } else {
    double c = 0.0;
    bool fin = true;
    for (int b = threadIdx.x; b < nmx; b += 256) {
      fin = fin && isfinite(aux[b]);
      c = fmax(c, aux[b]);
    }
    // same in every block; never warm after a failed orthogonality check
    const bool warm = __syncthreads_and(fin && c < 0.05 && st[ST_ROUNDS] == 0) != 0;
    if (warm) {
      for (int r = threadIdx.x; r < m; r += 256) V[(size_t)r * ld + j] = Wf[(size_t)r * ld + j];
    } else {
      for (int r = threadIdx.x; r < m; r += 256) S[(size_t)j * ld + r] = A[(size_t)j * ld + r];
    }
    if (j == 0 && threadIdx.x == 0) st[ST_PCJ] |= FLAG_FALLBACK | (warm ? 0 : FLAG_COLD);
  }
}

// ----------------------------------------------------------------------------
// Fallback: single-workgroup cyclic Jacobi on S (m x m fp64, global) with the
// eigenvectors accumulated in V; parallel round-robin ordering, each round
// applying up to m/2 disjoint rotations as 2x2 block updates. Runs only when
// the refinement did not converge.
__global__ __launch_bounds__(1024) void core_jacobi_kernel(double* S, double* V, int ld,
                                                           int32_t* st, double tol, int max_sweeps,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  V = iskv_rb(V, bdel);
  st = iskv_rb(st, bdel);
  if (!(st[ST_PCJ] & FLAG_FALLBACK)) return;
  __shared__ double cs[640], sn[640];
  __shared__ int pp[640], qq[640];
  __shared__ int active;
  const int n = st[ST_JM];
  const int t = threadIdx.x, nt = blockDim.x;
  if (st[ST_PCJ] & FLAG_COLD)
    for (int idx = t; idx < n * n; idx += nt) V[(size_t)(idx / n) * ld + idx % n] = (idx / n == idx % n) ? 1.0 : 0.0;
  __syncthreads();
  int sweep = 0;
  if (n >= 2) {
    const int N = (n + 1) & ~1, half = N / 2;
    for (; sweep < max_sweeps; ++sweep) {
      int rot_sweep = 0;
      for (int round = 0; round < N - 1; ++round) {
        if (t == 0) active = 0;
        __syncthreads();
        for (int i = t; i < half; i += nt) {
          int a = (i == 0) ? round % (N - 1) : (round + i) % (N - 1);
          int b = (i == 0) ? N - 1 : (round - i + (N - 1)) % (N - 1);
          int p = a < b ? a : b, q = a < b ? b : a;
          double c = 1.0, s = 0.0;
          if (q < n) {
            double app = S[(size_t)p * ld + p], aqq = S[(size_t)q * ld + q], apq = S[(size_t)p * ld + q];
            if (apq != 0.0 && fabs(apq) > tol * sqrt(fabs(app * aqq))) {
              rot2(app, aqq, apq, &c, &s);
              atomicAdd(&active, 1);
            }
          }
          cs[i] = c; sn[i] = s; pp[i] = p; qq[i] = q;
        }
        __syncthreads();
        if (active) {
          rot_sweep = 1;
          for (int blk = t; blk < half * half; blk += nt) {
            int a = blk / half, bb = blk % half;
            if (a > bb) continue;
            int pa = pp[a], qa = qq[a], pb = pp[bb], qb = qq[bb];
            if (qa >= n || qb >= n) continue;
            double ca = cs[a], sa = sn[a], cb = cs[bb], sb = sn[bb];
            if (sa == 0.0 && sb == 0.0) continue;
            double x11 = S[(size_t)pa * ld + pb], x12 = S[(size_t)pa * ld + qb];
            double x21 = S[(size_t)qa * ld + pb], x22 = S[(size_t)qa * ld + qb];
            double y11 = ca * x11 - sa * x21, y12 = ca * x12 - sa * x22;
            double y21 = sa * x11 + ca * x21, y22 = sa * x12 + ca * x22;
            double z11 = y11 * cb - y12 * sb, z12 = y11 * sb + y12 * cb;
            double z21 = y21 * cb - y22 * sb, z22 = y21 * sb + y22 * cb;
            if (a == bb) { z12 = 0.0; z21 = 0.0; }
            S[(size_t)pa * ld + pb] = z11; S[(size_t)pa * ld + qb] = z12;
            S[(size_t)qa * ld + pb] = z21; S[(size_t)qa * ld + qb] = z22;
            if (a != bb) {
              S[(size_t)pb * ld + pa] = z11; S[(size_t)qb * ld + pa] = z12;
              S[(size_t)pb * ld + qa] = z21; S[(size_t)qb * ld + qa] = z22;
            }
          }
          for (int e = t; e < n * half; e += nt) {
            int x = e / half, a = e % half;
            int p = pp[a], q = qq[a];
            if (q >= n) continue;
            double c = cs[a], s = sn[a];
            if (s == 0.0) continue;
            double vp = V[(size_t)x * ld + p], vq = V[(size_t)x * ld + q];
            V[(size_t)x * ld + p] = c * vp - s * vq;
            V[(size_t)x * ld + q] = s * vp + c * vq;
          }
        }
        __syncthreads();
      }
      if (!rot_sweep) break;
    }
  }
  if (t == 0) {
    st[ST_SWEEPS] = sweep;
    if (sweep >= max_sweeps) atomicOr(&st[ST_STATUS], ISKV_DEV_NOCONV);
  }
}

// ----------------------------------------------------------------------------
// Block Jacobi fallback for large cores (m_max > BJ_MIN_M). The indices are cut
// into blocks of 32; a round pairs the blocks (round-robin), and every pair of
// blocks is a 64 x 64 symmetric subproblem that one workgroup sweeps with
// cyclic Jacobi in LDS (BJ_INNER sweeps at most), accumulating its rotation Q. The pairs' rotations are
// disjoint, so S <- Q^T S Q and V <- V Q for the whole round are a row pass
// and a column pass over many workgroups. A sweep is NB - 1 rounds (NB blocks,
// even); the largest scaled coupling met in a sweep decides convergence.
constexpr int BJ_B = 32;          // block size
constexpr int BJ_P = 2 * BJ_B;    // pair size
constexpr int BJ_LD = BJ_P + 1;   // LDS row stride (doubles)
constexpr int BJ_NT = 512;        // threads of a pair solve (8 waves: two per SIMD)
constexpr int BJ_TW = 16;         // row / column tile of the row and column passes (16 or 32)
// Cores up to BJ_MIN_M keep the one-workgroup Jacobi: there the refinement
// converges except in early merges, and a merge's recorded sequence would
// otherwise carry the block Jacobi's ~1000 (mostly idle) launches.
constexpr int BJ_MIN_M = 384;
constexpr int BJ_SWEEPS = 32;
// Merges and re-orthogonalisations: the block Jacobi behind the refinement
// starts from the refinement's W when that is orthonormal and nearly
// converged, and needs at most 4 sweeps (cold) on the 64K-row r = 384 / 512
// streams; a recorded merge carries every sweep's launches, idle or not, so
// the budget is 12 rather than the dense solve's 32.
constexpr int BJ_SWEEPS_MERGE = 12;
#ifndef ISKV_BJ_INNER
#define ISKV_BJ_INNER 1
#endif
// Inner sweeps at most per pair subproblem. More than one measured no fewer
// outer sweeps on dense and clustered spectra (333-576), only slower merges
// (r = 512: 32 ms with one, 57 ms with up to eight).
constexpr int BJ_INNER = ISKV_BJ_INNER;
constexpr int FLAG_BJDONE = 8;
#ifndef ISKV_PCJ_MAXIT_LARGE
#define ISKV_PCJ_MAXIT_LARGE 3
#endif
constexpr int PCJ_MAXIT_LARGE = ISKV_PCJ_MAXIT_LARGE;

__device__ __forceinline__ bool bj_active(const int32_t* st) {
  const int f = st[ST_PCJ];
  return (f & FLAG_FALLBACK) && !(f & FLAG_BJDONE);
}

// Blocks of pair p in round r of a round-robin over NB blocks (NB even).
__device__ __forceinline__ void bj_pair(int r, int p, int NB, int* a, int* b) {
  const int x = p == 0 ? NB - 1 : (r + p) % (NB - 1);
  const int y = (r - p + NB - 1) % (NB - 1);
  *a = x < y ? x : y;
  *b = x < y ? y : x;
}

// Global index of local index l of the pair (blocks a, b).
__device__ __forceinline__ int bj_gidx(int l, int a, int b) { return l < BJ_B ? a * BJ_B + l : b * BJ_B + l - BJ_B; }

// The block Jacobi starts cold (FLAG_COLD: S = A, V = I) or from the
// refinement's last W (S = W^T A W and V = W, set by pcj_final only when W
// passed the orthonormality check and every coupling was below 0.05).
// smax[1] = max |a_ii|, the scale of the absolute part of the convergence
// test.
__global__ __launch_bounds__(256) void bj_init_kernel(const double* __restrict__ A, double* S, double* V, int ld,
                                                      int32_t* st, double* smax, const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  A = iskv_rb(A, bdel);
  S = iskv_rb(S, bdel);
  V = iskv_rb(V, bdel);
  st = iskv_rb(st, bdel);
  smax = iskv_rb(smax, bdel);
  if (!(st[ST_PCJ] & FLAG_FALLBACK)) return;
  const int m = st[ST_JM];
  if (blockIdx.x == 0) {
    __shared__ double red[4];
    double d = 0.0;
    for (int i = threadIdx.x; i < m; i += 256) d = fmax(d, fabs(A[(size_t)i * ld + i]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) d = fmax(d, __shfl_xor(d, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = d;
    __syncthreads();
    if (threadIdx.x == 0) {
      smax[0] = 0.0;
      smax[1] = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
      st[ST_SWEEPS] = 0;
    }
  }
  if (!(st[ST_PCJ] & FLAG_COLD)) return;
  const size_t tot = (size_t)m * m;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    const size_t i = e / m, j = e % m;
    S[i * ld + j] = A[i * ld + j];
    V[i * ld + j] = i == j ? 1.0 : 0.0;
  }
}

// bj_solve_kernel (after its helpers below): one cyclic sweep on the 64 x 64
// subproblem of pair p (grid.x) in round r;
// Q (64 x 64, row-major) to Qbuf[p]. The largest scaled coupling found,
// |s_ij| / max(sqrt(|s_ii s_jj|), 0.01 max_i |s_ii|) (relative, with an
// absolute floor at the rounding level of the largest entries), goes to
// smax[0] (atomic max on the bits of a non-negative double).
// A sweep is 63 rounds of 32 disjoint rotations in the round-robin order that
// keeps every round's pairs at positions (2k, 2k+1): A is held by position,
// and after a round the entry at positions (x, y) moves to (next(x), next(y))
// (bj_next), which brings every index back to its own position after the
// 63 rounds. Each wave forms the round's 32 rotations (a lane per pair, one
// division and one rsqrt each) and shares them through its own LDS row; then
// thread t takes pair column j = t % 32 and pair rows t / 32 + 16 u: it reads
// the 2 x 2 blocks of A at positions (2i, 2j) (bj_col: lanes read and write
// contiguous doubles), writes R_i^T A_ij R_j (the row rotation first) to the moved
// positions in the other copy of A, and applies R_j to the column pair at
// positions (2j, 2j+1) of rows t / 32 + 16 v of Q (also double-buffered: the
// columns move). One barrier per round, 8 waves (two per SIMD).

// The annihilating rotation of rot2 with one division: with d = aqq - app,
// t = sign(d) 2 apq / (|d| + sqrt(d^2 + 4 apq^2)) (tau = d / (2 apq) cleared
// from rot2's t = sign(tau) / (|tau| + sqrt(1 + tau^2))), c = 1 / sqrt(1 + t^2).
// For d = 0 either root t = +-1 annihilates; this takes sign(apq).
__device__ __forceinline__ void bj_rot2(double app, double aqq, double apq, double* c, double* s) {
  const double d = aqq - app;
  const double tt = (d >= 0.0 ? 2.0 : -2.0) * apq / (fabs(d) + sqrt(fma(d, d, 4.0 * apq * apq)));
  *c = rsqrt(fma(tt, tt, 1.0));
  *s = tt * (*c);
}

// Storage column of position x in a row of A or Q: even positions first
// (2j at column j), then odd ones (2j+1 at column 32 + j), so that a pair's
// two columns and their moved columns are each contiguous across lanes.
__device__ __forceinline__ int bj_col(int x) { return (x & 1) ? BJ_B + (x >> 1) : (x >> 1); }

__device__ __forceinline__ int bj_next(int x) {
  if (x == 0) return 0;
  if (x == 1) return 2;
  if ((x & 1) == 0) return x == BJ_P - 2 ? x + 1 : x + 2;
  return x - 2;
}

__global__ __launch_bounds__(BJ_NT) void bj_solve_kernel(const double* __restrict__ S, int ld, double* Qbuf,
                                                       int32_t* st, double* smax, int r, int NB, double tol,
                                                       const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  Qbuf = iskv_rb(Qbuf, bdel);
  st = iskv_rb(st, bdel);
  smax = iskv_rb(smax, bdel);
  if (!bj_active(st)) return;
  const int m = st[ST_JM];
  int a, b;
  bj_pair(r, blockIdx.x, NB, &a, &b);
  constexpr int BUF = BJ_P * BJ_LD;
  extern __shared__ double bj_lds[];
  double* Ab = bj_lds;            // [2][64][65]: A by position
  double* Qb = bj_lds + 2 * BUF;  // [2][64][65]: Q, columns by position
  __shared__ double red[BJ_NT / 64];
  const int t = threadIdx.x;
  double cmax = 0.0;
  const double floor_d = 0.01 * smax[1];
  for (int e = t; e < BJ_P * BJ_P; e += BJ_NT) {
    const int i = e / BJ_P, j = e % BJ_P;
    const int gi = bj_gidx(i, a, b), gj = bj_gidx(j, a, b);
    const double v = (gi < m && gj < m) ? S[(size_t)gi * ld + gj] : 0.0;
    Ab[i * BJ_LD + bj_col(j)] = v;
    Qb[i * BJ_LD + bj_col(j)] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int e = t; e < BJ_P * BJ_P; e += BJ_NT) {
    const int i = e / BJ_P, j = e % BJ_P;
    if (j > i) {
      const double den = fmax(sqrt(fabs(Ab[i * BJ_LD + bj_col(i)] * Ab[j * BJ_LD + bj_col(j)])), floor_d);
      const double x = fabs(Ab[i * BJ_LD + bj_col(j)]);
      const double c = !isfinite(x) ? INFINITY : (den > 0.0 ? x / den : (x > 0.0 ? INFINITY : 0.0));
      cmax = fmax(cmax, c);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cmax = fmax(cmax, __shfl_xor(cmax, o, 64));
  if ((t & 63) == 0) red[t >> 6] = cmax;
  __syncthreads();
  if (t == 0) {
    double c = 0.0;
    for (int w = 0; w < BJ_NT / 64; ++w) c = fmax(c, red[w]);
    atomicMax((unsigned long long*)smax, (unsigned long long)__double_as_longlong(c));
  }
  constexpr int IST = BJ_NT / BJ_B;  // pair rows (and Q rows) step between a thread's blocks
  const int jj = t & (BJ_B - 1), i0 = t / BJ_B, lane = t & 63, wave = t >> 6;
  const int nj0 = bj_col(bj_next(2 * jj)), nj1 = bj_col(bj_next(2 * jj + 1));
  __shared__ double csw[BJ_NT / 64][BJ_B], snw[BJ_NT / 64][BJ_B];
  __shared__ int rotated;
  int cur = 0;
  for (int inner = 0; inner < BJ_INNER; ++inner) {
    if (t == 0) rotated = 0;
    __syncthreads();
    bool rot_any = false;
    for (int rr = 0; rr < BJ_P - 1; ++rr) {
      const double* A = Ab + cur * BUF;
      double* An = Ab + (cur ^ 1) * BUF;
      const double* Qc = Qb + cur * BUF;
      double* Qn = Qb + (cur ^ 1) * BUF;
      // the round's rotations (pair k at positions 2k, 2k+1), the same
      // arithmetic in every wave; the wave's LDS operations complete in
      // order, and the fence keeps the compiler from moving them
      if (lane < BJ_B) {
        const int p = 2 * lane, q = p + 1;
        const double app = A[p * BJ_LD + lane], aqq = A[q * BJ_LD + BJ_B + lane], apq = A[p * BJ_LD + BJ_B + lane];
        double c = 1.0, sv = 0.0;
        if (apq != 0.0 && isfinite(apq) && fabs(apq) > tol * sqrt(fabs(app * aqq))) {
          bj_rot2(app, aqq, apq, &c, &sv);
          rot_any = true;
        }
        csw[wave][lane] = c;
        snw[wave][lane] = sv;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // every operand of the round is read before any result is written (the
      // two copies share one LDS array, so a store would otherwise hold back
      // the loads after it)
      const double cj = csw[wave][jj], sj = snw[wave][jj];
      constexpr int UA = BJ_B / IST, VQ = BJ_P / IST;
      double ci[UA], si[UA], x[UA][4], vq[VQ][2];
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int i = i0 + IST * u;
        ci[u] = csw[wave][i];
        si[u] = snw[wave][i];
        x[u][0] = A[(2 * i) * BJ_LD + jj];
        x[u][1] = A[(2 * i) * BJ_LD + BJ_B + jj];
        x[u][2] = A[(2 * i + 1) * BJ_LD + jj];
        x[u][3] = A[(2 * i + 1) * BJ_LD + BJ_B + jj];
      }
#pragma unroll
      for (int v = 0; v < VQ; ++v) {
        const int row = i0 + IST * v;
        vq[v][0] = Qc[row * BJ_LD + jj];
        vq[v][1] = Qc[row * BJ_LD + BJ_B + jj];
      }
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int i = i0 + IST * u;
        const double y11 = ci[u] * x[u][0] - si[u] * x[u][2], y21 = si[u] * x[u][0] + ci[u] * x[u][2];
        const double y12 = ci[u] * x[u][1] - si[u] * x[u][3], y22 = si[u] * x[u][1] + ci[u] * x[u][3];
        const int ni0 = bj_next(2 * i), ni1 = bj_next(2 * i + 1);
        An[ni0 * BJ_LD + nj0] = cj * y11 - sj * y12;
        An[ni0 * BJ_LD + nj1] = sj * y11 + cj * y12;
        An[ni1 * BJ_LD + nj0] = cj * y21 - sj * y22;
        An[ni1 * BJ_LD + nj1] = sj * y21 + cj * y22;
      }
#pragma unroll
      for (int v = 0; v < VQ; ++v) {
        const int row = i0 + IST * v;
        Qn[row * BJ_LD + nj0] = cj * vq[v][0] - sj * vq[v][1];
        Qn[row * BJ_LD + nj1] = sj * vq[v][0] + cj * vq[v][1];
      }
      cur ^= 1;
      __syncthreads();
    }
    if (rot_any) rotated = 1;
    __syncthreads();
    // every thread reads the flag before thread 0 may clear it for the next
    // sweep, so the exit is uniform across the workgroup
    const int any = rotated;
    __syncthreads();
    if (!any) break;
  }
  // whole sweeps only: every index is back at its own position
  const double* Qf = Qb + cur * BUF;
  double* Qo = Qbuf + (size_t)blockIdx.x * BJ_P * BJ_P;
  for (int e = t; e < BJ_P * BJ_P; e += BJ_NT) Qo[e] = Qf[(e / BJ_P) * BJ_LD + bj_col(e % BJ_P)];
}

// Row pass: S[I, j0 .. j0+BJ_TW) <- Q^T S[I, j0 .. j0+BJ_TW) for the pair's 64
// indices I, on the fp64 matrix cores. Grid (pairs, column tiles).
__global__ __launch_bounds__(256) void bj_rows_kernel(double* S, int ld, const double* __restrict__ Qbuf,
                                                      const int32_t* st, int r, int NB,
                                                      const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  Qbuf = iskv_rb(Qbuf, bdel);
  st = iskv_rb(st, bdel);
  if (!bj_active(st)) return;
  const int m = st[ST_JM];
  const int j0 = blockIdx.y * BJ_TW;
  if (j0 >= m) return;
  int a, b;
  bj_pair(r, blockIdx.x, NB, &a, &b);
  __shared__ double Qs[BJ_P][BJ_LD], X[BJ_P][BJ_TW + 1];
  const double* Qp = Qbuf + (size_t)blockIdx.x * BJ_P * BJ_P;
  const int t = threadIdx.x;
  for (int e = t; e < BJ_P * BJ_P; e += 256) Qs[e / BJ_P][e % BJ_P] = Qp[e];
  for (int e = t; e < BJ_P * BJ_TW; e += 256) {
    const int i = e / BJ_TW, j = e % BJ_TW;
    const int gi = bj_gidx(i, a, b), gj = j0 + j;
    X[i][j] = (gi < m && gj < m) ? S[(size_t)gi * ld + gj] : 0.0;
  }
  __syncthreads();
  // wave w: output rows 16 w .. 16 w + 15 and the tile's columns, as 16 x 16
  // tiles on v_mfma_f64_16x16x4f64 (lane layout as in dgemm_kernel)
  const int lane = t & 63, w = t >> 6, rl = lane & 15, g = lane >> 4;
  constexpr int TPW = BJ_TW / 16;  // 16 x 16 tiles per wave
  v4d acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int kk = 0; kk < BJ_P / 4; ++kk) {
    const double av = Qs[4 * kk + g][16 * w + rl];  // (Q^T)[16 w + rl][4 kk + g]
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, X[4 * kk + g][16 * u + rl], acc[u], 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + g + 4 * e, j = 16 * u + rl;
      const int gi = bj_gidx(i, a, b), gj = j0 + j;
      if (gi < m && gj < m) S[(size_t)gi * ld + gj] = acc[u][e];
    }
  }
}

// Column pass: S[i, I] <- S[i, I] Q and V[i, I] <- V[i, I] Q for rows
// i0 .. i0+BJ_TW-1, on the fp64 matrix cores. Grid (pairs, row tiles).
__global__ __launch_bounds__(256) void bj_cols_kernel(double* S, double* V, int ld, const double* __restrict__ Qbuf,
                                                      const int32_t* st, int r, int NB,
                                                      const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  V = iskv_rb(V, bdel);
  Qbuf = iskv_rb(Qbuf, bdel);
  st = iskv_rb(st, bdel);
  if (!bj_active(st)) return;
  const int m = st[ST_JM];
  const int i0 = blockIdx.y * BJ_TW;
  if (i0 >= m) return;
  int a, b;
  bj_pair(r, blockIdx.x, NB, &a, &b);
  // Q and both row tiles are staged at once, so their loads are in flight together
  __shared__ double Qs[BJ_P][BJ_LD], X[2][BJ_TW][BJ_LD];
  const double* Qp = Qbuf + (size_t)blockIdx.x * BJ_P * BJ_P;
  const int t = threadIdx.x;
  for (int e = t; e < BJ_P * BJ_P; e += 256) Qs[e / BJ_P][e % BJ_P] = Qp[e];
  for (int e = t; e < BJ_TW * BJ_P; e += 256) {
    const int i = e / BJ_P, j = e % BJ_P;
    const int gi = i0 + i, gj = bj_gidx(j, a, b);
    const bool in = gi < m && gj < m;
    X[0][i][j] = in ? S[(size_t)gi * ld + gj] : 0.0;
    X[1][i][j] = in ? V[(size_t)gi * ld + gj] : 0.0;
  }
  __syncthreads();
  // the tile's rows of X Q as 16 x 16 MFMA tiles, the same number per wave
  const int lane = t & 63, w = t >> 6, rl = lane & 15, g = lane >> 4;
  constexpr int TPW = BJ_TW / 16;  // 16 x 16 tiles per wave
  const int rw = 16 * (w % TPW), cu = TPW * (w / TPW);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    double* M = pass == 0 ? S : V;
    v4d acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = v4d{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
    for (int kk = 0; kk < BJ_P / 4; ++kk) {
      const double av = X[pass][rw + rl][4 * kk + g];
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, Qs[4 * kk + g][16 * (cu + u) + rl], acc[u], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = i0 + rw + g + 4 * e, gj = bj_gidx(16 * (cu + u) + rl, a, b);
        if (gi < m && gj < m) M[(size_t)gi * ld + gj] = acc[u][e];
      }
    }
  }
}

// End of a sweep: converged when the sweep's largest scaled coupling is below
// tol; after the last sweep, no convergence is reported in the status.
__global__ void bj_check_kernel(int32_t* st, double* smax, double tol, int last,
                                const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  st = iskv_rb(st, bdel);
  smax = iskv_rb(smax, bdel);
  if (!bj_active(st)) return;
  st[ST_SWEEPS] += 1;
  if (smax[0] < tol) st[ST_PCJ] |= FLAG_BJDONE;
  else if (last) atomicOr(&st[ST_STATUS], ISKV_DEV_NOCONV);
  smax[0] = 0.0;
}

inline size_t bj_lds_bytes() { return (size_t)4 * BJ_P * BJ_LD * sizeof(double); }

// A dense matrix goes straight to the block Jacobi (cold: S = A, V = I).
__global__ void bj_force_kernel(int32_t* st) {
  st[ST_PCJ] = FLAG_FALLBACK | FLAG_COLD;
  st[ST_PCJIT] = 0;
  st[ST_ROUNDS] = 0;
}
// Sweep budget of a dense solve (enqueued up front; sweeps after convergence
// return at once).
constexpr int BJ_SWEEPS_DENSE = 16;

}  // namespace

void iskv_dgemm(hipStream_t s, int m_max, const double* A, bool ta, const double* B, bool tb, double* C,
                const double* Cin, int ld, double alpha, double beta, double gamma, const int32_t* st,
                int mode, const int64_t* bd, int bc) {
  if (!ta && !tb) gemm<false, false>(s, m_max, A, B, C, Cin, ld, alpha, beta, gamma, st, mode, bd, bc);
  else if (ta && !tb) gemm<true, false>(s, m_max, A, B, C, Cin, ld, alpha, beta, gamma, st, mode, bd, bc);
  else if (!ta && tb) gemm<false, true>(s, m_max, A, B, C, Cin, ld, alpha, beta, gamma, st, mode, bd, bc);
  else gemm<true, true>(s, m_max, A, B, C, Cin, ld, alpha, beta, gamma, st, mode, bd, bc);
}

int iskv_core_eig_setup() {
  ISKV_HIP_CHECK(hipFuncSetAttribute((const void*)bgemm2_kernel<true, true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bt_lds_bytes(true)));
  ISKV_HIP_CHECK(hipFuncSetAttribute((const void*)bgemm2_kernel<false, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bt_lds_bytes(true)));
  ISKV_HIP_CHECK(hipFuncSetAttribute((const void*)pcj_analyze_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)sizeof(AnalyzeLds)));
  ISKV_HIP_CHECK(hipFuncSetAttribute((const void*)bj_solve_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)bj_lds_bytes()));
  return ISKV_OK;
}

// Eigen-decompose the m x m matrix in w.A (m = st[ST_JM]): on return the
// diagonal of w.S holds the eigenvalues and w.V the eigenvectors (columns),
// unsorted. Fixed launch sequence; no host synchronisation.
int iskv_launch_core_eig(isvd_handle* h, double tol, int keep) {
  const isvd_ws& w = h->w;
  hipStream_t s = h->stream;
  const int mm = h->m_max, ld = h->ldm;
  int32_t* st = w.st;
  const int nblk = (mm + 15) / 16;
  const size_t lds = sizeof(AnalyzeLds);
  const int NB = ((mm + BJ_B - 1) / BJ_B + 1) & ~1;
  const int tiles = (mm + BJ_TW - 1) / BJ_TW;
  // block Jacobi: Km (free once the refinement has ended) holds the pairs'
  // rotations, aux[0] the sweep's largest coupling
  auto block_jacobi = [&](int sweeps) {
    hipLaunchKernelGGL(bj_init_kernel, bz(dim3(64), h->bcount), dim3(256), 0, s, w.A, w.S, w.V, ld, st, w.aux,
                       h->bd);
    for (int sw = 0; sw < sweeps; ++sw) {
      for (int r = 0; r < NB - 1; ++r) {
        hipLaunchKernelGGL(bj_solve_kernel, bz(dim3(NB / 2), h->bcount), dim3(BJ_NT), bj_lds_bytes(), s, w.S, ld, w.Km,
                           st, w.aux, r, NB, 1e-13, h->bd);
        hipLaunchKernelGGL(bj_rows_kernel, bz(dim3(NB / 2, tiles), h->bcount), dim3(256), 0, s, w.S, ld, w.Km, st, r,
                           NB, h->bd);
        hipLaunchKernelGGL(bj_cols_kernel, bz(dim3(NB / 2, tiles), h->bcount), dim3(256), 0, s, w.S, w.V, ld, w.Km, st,
                           r, NB, h->bd);
      }
      // converged at the solve's tolerance (at least 1e-10: the two 64-term
      // passes leave ~1e-14 max|s_ii| of rounding in the entries, scaled
      // couplings near 1e-12 at the absolute floor)
      hipLaunchKernelGGL(bj_check_kernel, bz(dim3(1), h->bcount), dim3(1), 0, s, st, w.aux, fmax(tol, 1e-10),
                         sw == sweeps - 1 ? 1 : 0, h->bd);
    }
  };
  const bool bj_fits = (size_t)(NB / 2) * BJ_P * BJ_P <= (size_t)ld * ld && w.naux >= 2;
  if (h->force_block_jacobi && bj_fits && h->bcount == 1) {
    // a dense matrix (the refit's Rayleigh-Ritz core): no refinement
    hipLaunchKernelGGL(bj_force_kernel, dim3(1), dim3(1), 0, s, st);
    block_jacobi(BJ_SWEEPS_DENSE);
    ISKV_HIP_CHECK(hipGetLastError());
    return ISKV_OK;
  }
  hipLaunchKernelGGL(pcj_init_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.A, w.S, w.W0, ld, st, h->bd);
  // step 0 works on S = A with W = I
  hipLaunchKernelGGL(pcj_detect_kernel, bz(dim3(nblk, nblk), h->bcount), dim3(256), 0, s, w.S, ld, w.aux, w.edges,
                     st, tol, keep, h->bd);
  hipLaunchKernelGGL(pcj_analyze_kernel, bz(dim3(1), h->bcount), dim3(1024), lds, s, w.S, ld, w.aux, nblk * nblk,
                     w.edges, w.itab, w.rtab, h->m_max, st, 0, tol, h->bd);
  hipLaunchKernelGGL(pcj_kmat_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.S, ld, w.Km, w.Pa, w.W0, w.itab,
                     w.rtab, h->m_max, st, h->bd);
  // X = I + K (I + K/2); W <- W X
  gemm<false, false>(s, mm, w.Km, w.Pa, w.Pb, nullptr, ld, 1.0, 0.0, 1.0, st, 0, h->bd, h->bcount);
  gemm<false, false>(s, mm, w.W0, w.Pb, w.W1, w.W0, ld, 1.0, 0.0, 0.0, st, 1, h->bd, h->bcount);
  // From step 1 on, W sits in `wc` at the start of a step and its
  // re-orthonormalised form W' in `wo`; after convergence `wo` keeps the final
  // W (the launches that would change it are skipped).
  double* wc = w.W1;
  double* wo = w.W0;
  // cores above BJ_MIN_M rarely converge in the refinement (flat spectral
  // floors) and have the block Jacobi behind them: fewer steps there
  const int maxit = mm > BJ_MIN_M ? PCJ_MAXIT_LARGE : PCJ_MAXIT;
  for (int it = 1; it <= maxit; ++it) {
    // T1 = W^T W and T2 = A W (A symmetric: read as A^T)
    gemm2<true, true>(s, mm, wc, w.A, wc, ld, w.T, w.Km, nullptr, nullptr, 1.0, 0.0, 1.0, 0.0, nullptr, st, 0, h->bd,
                      h->bcount);
    // Newton-Schulz W' = 1.5 W - 0.5 W T1, and A W' = 1.5 T2 - 0.5 T2 T1 (keeps W
    // orthonormal to O(defect^2), so S is measured in an orthonormal basis);
    // partial sums of diag(W'^T A W')
    gemm2<false, false>(s, mm, wc, w.Km, w.T, ld, wo, w.Pa, wc, w.Km, -0.5, 1.5, -0.5, 1.5, w.Dp, st, 0, h->bd,
                        h->bcount);
    // S = W'^T (A W') with the strong-pair detection
    gemm_s(s, mm, wo, w.Pa, ld, w.S, w.Dp, w.aux, w.edges, st, tol, h->bd, h->bcount);
    hipLaunchKernelGGL(pcj_analyze_kernel, bz(dim3(1), h->bcount), dim3(1024), lds, s, w.S, ld, w.aux,
                       nblk * nblk, w.edges, w.itab, w.rtab, h->m_max, st, it, tol, h->bd);
    if (it == maxit) break;  // last pass only tests convergence
    hipLaunchKernelGGL(pcj_kmat_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.S, ld, w.Km, w.Pa, wo, w.itab,
                       w.rtab, h->m_max, st, h->bd);
    gemm<false, false>(s, mm, w.Km, w.Pa, w.Pb, nullptr, ld, 1.0, 0.0, 1.0, st, 0, h->bd, h->bcount);
    gemm<false, false>(s, mm, wo, w.Pb, wc, wo, ld, 1.0, 0.0, 0.0, st, 1, h->bd, h->bcount);
  }
  // final Newton-Schulz of W (in wo) into wc, with A W for the eigenvalues;
  // skipped after convergence at a step >= 1 when the iterate behind wo was
  // within 1e-4 of orthonormal (wo then within ~1e-8, Pa = A wo, and T keeps
  // W^T W of that iterate)
  hipLaunchKernelGGL(pcj_orth_check_kernel, bz(dim3(64), h->bcount), dim3(256), 0, s, w.T, ld, st, 1e-4, 1, h->bd);
  gemm2<true, true>(s, mm, wo, w.A, wo, ld, w.T, w.Km, nullptr, nullptr, 1.0, 0.0, 1.0, 0.0, nullptr, st, 4, h->bd,
                    h->bcount);
  gemm2<false, false>(s, mm, wo, w.Km, w.T, ld, wc, w.Pa, wo, w.Km, -0.5, 1.5, -0.5, 1.5, nullptr, st, 4, h->bd,
                      h->bcount);
  hipLaunchKernelGGL(pcj_orth_check_kernel, bz(dim3(64), h->bcount), dim3(256), 0, s, w.T, ld, st, 1e-4, 0, h->bd);
  // S = W^T A W of the final W, used only by a fallback that continues from it
  gemm<true, false>(s, mm, wc, w.Pa, w.S, nullptr, ld, 1.0, 0.0, 0.0, st, 3, h->bd, h->bcount);
  hipLaunchKernelGGL(pcj_final_kernel, bz(dim3(mm), h->bcount), dim3(256), 0, s, wo, wc, w.Pa, w.A, w.S, w.V, ld,
                     w.aux, nblk * nblk, st, h->bd);
  if (!bj_fits || mm <= BJ_MIN_M) {
    hipLaunchKernelGGL(core_jacobi_kernel, bz(dim3(1), h->bcount), dim3(1024), 0, s, w.S, w.V, ld, st, 1e-13,
                       ISKV_JACOBI_MAX_SWEEPS, h->bd);
  } else {
    block_jacobi(keep >= 0 ? BJ_SWEEPS_MERGE : BJ_SWEEPS);
  }
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}
