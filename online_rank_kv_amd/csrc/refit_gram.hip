// Fresh rank-k truncated SVD of n given rows X (n x D, fp32) on the GPU: the
// factor of Algorithm 1 (the non-exact prompt rows) and of the value first
// refit of §3.2 in the iS-KV notes, where the history is rebuilt from scratch
// rather than folded block by block.
//
// The rank-k truncated SVD of X is X B B^T with B the top-k eigenvectors of
// the Gram G = X^T X (D x D). Route on gfx950:
//   1. G in fp64 on the matrix cores (products of fp32 entries are exact in
//      fp64, so G carries only the fp64 rounding of its sums);
//   2. subspace iteration on G with an oversampled block of l = min(D, r + b)
//      columns: V <- orth(G V), `iters` times. The angle between span(V) and
//      the top-k eigenspace shrinks by lambda_{l+1} / lambda_k per step, so
//      the oversampling (b columns beyond the rank) makes the rate
//      independent of the gap at the cut, which is tiny on flat spectra;
//   3. Rayleigh-Ritz: the eigendecomposition of the l x l matrix V^T G V
//      (the handle's core eigensolver), whose top k eigenvectors W give
//      B = V W[:, :k] and the singular values sqrt(theta_j);
//   4. C = X B (C^T C = B^T G B = diag(theta): orthogonal columns with norms
//      sigma, the state every later merge assumes).
// orth() is CholeskyQR in fp64 on the column-normalised Y: with
// S = diag(1/|y_j|), S Y^T Y S + s I = L L^T (blocked, 64-wide panels: one
// launch factors the diagonal block and solves the panel below it, one GEMM
// updates the trailing matrix), then V = Y S L^-T. With V orthonormal,
// Y = G V has condition at most about cond(G); the tiny relative shift s
// keeps a rank-deficient Y factorable, and the normalisation makes a
// dependent column come out as an orthonormal rounding direction (harmless
// to Rayleigh-Ritz) instead of a tiny skewed one. The block is capped at n
// columns: n rows span at most n directions. The last basis gets a second
// pass (CholeskyQR2) before the Ritz step.
#include "iskv_internal.h"

#include <math.h>

#include <utility>

namespace {

typedef double v4d_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double ld_elt(const double* p) { return *p; }
__device__ __forceinline__ double ld_elt(const float* p) { return (double)*p; }

// C (M x N, ldc) = alpha op(A) op(B) + beta C, fp64 on the matrix cores
// (v_mfma_f64_16x16x4f64; A fragment: lane l holds A[l % 16][l / 16], B
// fragment: B[l / 16][l % 16], result lane l element e: C[l / 16 + 4 e][l % 16]).
// op(A) is M x K: A stored M x K (lda), or K x M when TA. op(B) is K x N: B
// stored K x N (ldb), or N x K when TB. Element types TEA / TEB are float or
// double (widened exactly). A 256-thread workgroup owns a 64 x 64 tile; wave
// w computes its 32 x 32 quarter as 2 x 2 blocks; K goes in steps of 64
// (four chunks of 16) staged in LDS, the next step's loads in flight during
// the current one, so the K = 64 products of the Cholesky panels and the
// triangular solves take one step.
// lower_only: tiles strictly above the diagonal are skipped. beta == 0 never
// reads C. C may be the A operand itself when N <= 64 (one tile column): a
// workgroup reads all of its rows of A before it writes any of them.
constexpr int RG_T = 64, RG_KC = 16, RG_LS = RG_T + 4;
constexpr int RG_NCH = 4;  // 16-deep chunks staged per step (64 of K: one step for the K = 64 panel products)

template <bool TA, bool TB, typename TEA, typename TEB>
__global__ __launch_bounds__(256) void rg_gemm_kernel(const TEA* A, int lda, const TEB* B, int ldb, double* C, int ldc,
                                                      int M, int N, int K, double alpha, double beta, int lower_only) {
  const int i0 = blockIdx.y * RG_T, j0 = blockIdx.x * RG_T;
  if (lower_only && j0 > i0) return;
  __shared__ double As[RG_NCH][RG_KC][RG_LS], Bs[RG_NCH][RG_KC][RG_LS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  double ar[RG_NCH][4], br[RG_NCH][4];
  // staging map: TA / !TB chunks are read along rows of 64 (k = t / 16,
  // 4 consecutive entries from 4 (t % 16)); !TA / TB along rows of 16
  // (entry = t / 4, 4 consecutive k from 4 (t % 4))
  auto load = [&](int k0s) {
#pragma unroll
    for (int ch = 0; ch < RG_NCH; ++ch) {
    const int k0 = k0s + RG_KC * ch;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (TA) {
        const int kk = t >> 4, i = ((t & 15) << 2) + q;
        const bool in = k0 + kk < K && i0 + i < M;
        ar[ch][q] = in ? ld_elt(A + (size_t)(k0 + kk) * lda + i0 + i) : 0.0;
      } else {
        const int i = t >> 2, kk = ((t & 3) << 2) + q;
        const bool in = k0 + kk < K && i0 + i < M;
        ar[ch][q] = in ? ld_elt(A + (size_t)(i0 + i) * lda + k0 + kk) : 0.0;
      }
      if (TB) {
        const int j = t >> 2, kk = ((t & 3) << 2) + q;
        const bool in = k0 + kk < K && j0 + j < N;
        br[ch][q] = in ? ld_elt(B + (size_t)(j0 + j) * ldb + k0 + kk) : 0.0;
      } else {
        const int kk = t >> 4, j = ((t & 15) << 2) + q;
        const bool in = k0 + kk < K && j0 + j < N;
        br[ch][q] = in ? ld_elt(B + (size_t)(k0 + kk) * ldb + j0 + j) : 0.0;
      }
    }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int ch = 0; ch < RG_NCH; ++ch)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (TA) As[ch][t >> 4][((t & 15) << 2) + q] = ar[ch][q];
      else As[ch][((t & 3) << 2) + q][t >> 2] = ar[ch][q];
      if (TB) Bs[ch][((t & 3) << 2) + q][t >> 2] = br[ch][q];
      else Bs[ch][t >> 4][((t & 15) << 2) + q] = br[ch][q];
    }
  };
  v4d_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = v4d_t{0.0, 0.0, 0.0, 0.0};
  if (K > 0) load(0);
  for (int k0 = 0; k0 < K; k0 += RG_NCH * RG_KC) {
    __syncthreads();
    store();
    __syncthreads();
    if (k0 + RG_NCH * RG_KC < K) load(k0 + RG_NCH * RG_KC);
#pragma unroll
    for (int k4 = 0; k4 < 4 * RG_NCH; ++k4) {
      const int ch = k4 >> 2, kk = 4 * (k4 & 3) + (lane >> 4);
      double av[2], bv[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) av[a] = As[ch][kk][32 * wr + 16 * a + (lane & 15)];
#pragma unroll
      for (int b = 0; b < 2; ++b) bv[b] = Bs[ch][kk][32 * wc + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 32 * wr + 16 * a + (lane >> 4) + 4 * e;
        const int j = j0 + 32 * wc + 16 * b + (lane & 15);
        if (i < M && j < N) {
          double o = alpha * acc[a][b][e];
          if (beta != 0.0) o += beta * C[(size_t)i * ldc + j];
          C[(size_t)i * ldc + j] = o;
        }
      }
}

template <bool TA, bool TB, typename TEA, typename TEB>
void rg_gemm(hipStream_t s, const TEA* A, int lda, const TEB* B, int ldb, double* C, int ldc, int M, int N, int K,
             double alpha, double beta, bool lower_only = false) {
  if (M <= 0 || N <= 0) return;
  dim3 grid((N + RG_T - 1) / RG_T, (M + RG_T - 1) / RG_T);
  hipLaunchKernelGGL((rg_gemm_kernel<TA, TB, TEA, TEB>), grid, dim3(256), 0, s, A, lda, B, ldb, C, ldc, M, N, K,
                     alpha, beta, lower_only ? 1 : 0);
}

// Random start basis: V[d][j] uniform in [-1, 1) from a splitmix64 hash of
// (d, j) (a fixed stream: the refit is deterministic).
__global__ __launch_bounds__(256) void rg_rand_kernel(double* V, int D, int l) {
  const size_t tot = (size_t)D * l;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    unsigned long long z = e + 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    V[e] = 2.0 * ((double)(z >> 11) * (1.0 / 9007199254740992.0)) - 1.0;
  }
}

// Column scaling of the Cholesky input: rs[j] = 1 / sqrt(M[j][j]) (0 for a
// zero column), so that the scaled Gram diag(rs) M diag(rs) has a unit
// diagonal. CholeskyQR on the normalised columns of Y keeps every column's
// independent part at its own scale: a column that depends on the earlier
// ones to rounding comes out as a rounding direction that the next pass
// normalises, never as a tiny, skewed column.
__global__ __launch_bounds__(256) void rg_diag_kernel(const double* __restrict__ A, int ld, int m, double* rs) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < m) {
    const double d = A[(size_t)j * ld + j];
    rs[j] = d > 0.0 ? 1.0 / sqrt(d) : 0.0;
  }
}

// A <- diag(rs) A diag(rs) + shift I over the m x m block (the shift is the
// pivot floor of the Cholesky, relative to the unit diagonal).
__global__ __launch_bounds__(256) void rg_scale_kernel(double* A, int ld, int m, const double* __restrict__ rs,
                                                       double shift) {
  const size_t tot = (size_t)m * m;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    const int i = (int)(e / m), j = (int)(e % m);
    double v = A[(size_t)i * ld + j] * rs[i] * rs[j];
    if (i == j) v += shift;
    A[(size_t)i * ld + j] = v;
  }
}

// Diagonal block of panel j0 of the right-looking Cholesky M = L L^T (one
// workgroup, in LDS): factor the 64 x 64 block (already updated by the
// earlier panels) and invert its factor. Every phase keeps its dependency
// chains in registers, so that LDS round trips do not serialise:
// - elimination in the unscaled form (step c subtracts a[r][c] a[q][c] / p_c
//   from every trailing entry, p_c = max(a[c][c], floor_)) in four
//   16-column steps: wave 0 holds the 16 x 16 diagonal block as a full
//   symmetric square in registers (lane 4 rr + g: row rr, columns 4 g..4 g+3)
//   and eliminates it column by column with cross-lane reads; then a thread
//   per row solves the panel below it from its 16 entries in registers, and
//   the workgroup updates the trailing lower triangle;
// - L[r][c] = a[r][c] / sqrt(p_c), stored back into M;
// - X = L^-1 (lower) by doubling: the four 16 x 16 diagonal blocks by forward
//   substitution (a thread per column, the column in registers), then pairs
//   of blocks with [[A, 0], [B, C]]^-1 = [[A^-1, 0], [-C^-1 B A^-1, C^-1]] at
//   sizes 16 and 32, each off-diagonal block as two workgroup-wide products;
//   X goes to Li.
// Rows and columns past m are identity padding.
constexpr int RG_CB = 64;
constexpr int RG_CS = RG_CB + 1;  // LDS row stride: a column walk spreads over the banks

__global__ __launch_bounds__(256) void rg_chol_diag_kernel(double* A, int ld, int m, int j0, double floor_,
                                                           double* Li) {
  __shared__ double Lu[RG_CB * RG_CS];
  __shared__ double X[RG_CB * RG_CS];
  __shared__ double Tb[32 * 32];  // B A^-1 of the doubling step
  __shared__ double ip[RG_CB];    // 1 / p_c
  const int t = threadIdx.x, lane = t & 63;
  const int nb = min(RG_CB, m - j0);
  const int q = t & 63, r0 = t >> 6;
  // the lower triangle (the upper one is never read); X starts at zero
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = r0 + 4 * u;
    double v = 0.0;
    if (r < nb && q <= r) v = A[(size_t)(j0 + r) * ld + j0 + q];
    if (r >= nb && r == q) v = 1.0;
    Lu[r * RG_CS + q] = v;
    X[r * RG_CS + q] = 0.0;
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < RG_CB; o += 16) {
    if (t < 64) {
      const int rr = lane >> 2, g = lane & 3;
      double a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cc = 4 * g + j;
        a[j] = cc <= rr ? Lu[(o + rr) * RG_CS + o + cc] : Lu[(o + cc) * RG_CS + o + rr];
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        // pivot a[c][c] (lane 4 c + c / 4), a[rr][c] (lane 4 rr + c / 4) and
        // a[c][4 g + j] = a[4 g + j][c] (lane 4 c + g), all from slot c % 4
        // or j, read before this column's update
        const double dcc = a[c & 3];
        const int lo = __builtin_amdgcn_readlane((int)__double2loint(dcc), 4 * c + (c >> 2));
        const int hi = __builtin_amdgcn_readlane((int)__double2hiint(dcc), 4 * c + (c >> 2));
        const double inv = 1.0 / fmax(__hiloint2double(hi, lo), floor_);
        const double arc = __shfl(dcc, 4 * rr + (c >> 2));
        double acq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acq[j] = __shfl(a[j], 4 * c + g);
        if (lane == 0) ip[o + c] = inv;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (rr > c && 4 * g + j > c) a[j] = fma(-(arc * acq[j]), inv, a[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * g + j <= rr) Lu[(o + rr) * RG_CS + o + 4 * g + j] = a[j];
    }
    __syncthreads();
    if (o + 16 < RG_CB) {
      // the panel below the block: row r, columns o..o+15
      if (t < RG_CB - o - 16) {
        const int r = o + 16 + t;
        double x[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = Lu[r * RG_CS + o + k];
#pragma unroll
        for (int c = 1; c < 16; ++c) {
          double s0 = x[c], s1 = 0.0;
#pragma unroll
          for (int k = 0; k < c; ++k) {
            const double f = Lu[(o + c) * RG_CS + o + k] * ip[o + k];
            if (k & 1) s1 = fma(-x[k], f, s1);
            else s0 = fma(-x[k], f, s0);
          }
          x[c] = s0 + s1;
        }
#pragma unroll
        for (int k = 1; k < 16; ++k) Lu[r * RG_CS + o + k] = x[k];
      }
      __syncthreads();
      // the trailing lower triangle
      const int w2 = RG_CB - o - 16;
      for (int e = t; e < w2 * w2; e += 256) {
        const int r = o + 16 + e / w2, qq = o + 16 + e % w2;
        if (qq > r) continue;
        double s0 = Lu[r * RG_CS + qq], s1 = 0.0;
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          s0 = fma(-(Lu[r * RG_CS + o + k] * Lu[qq * RG_CS + o + k]), ip[o + k], s0);
          s1 = fma(-(Lu[r * RG_CS + o + k + 1] * Lu[qq * RG_CS + o + k + 1]), ip[o + k + 1], s1);
        }
        Lu[r * RG_CS + qq] = s0 + s1;
      }
      __syncthreads();
    }
  }
  // L = column-scaled factor (lower), kept in Lu and stored to M
  {
    const double dq = sqrt(fmax(Lu[q * RG_CS + q], floor_));
    const double rq = 1.0 / dq;
    double v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = r0 + 4 * u;
      v[u] = q < r ? Lu[r * RG_CS + q] * rq : (q == r ? dq : 0.0);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = r0 + 4 * u;
      Lu[r * RG_CS + q] = v[u];
      if (r < nb && q <= r) A[(size_t)(j0 + r) * ld + j0 + q] = v[u];
    }
    __syncthreads();
  }
  // the four diagonal 16 x 16 blocks of X, a thread per column j (the zeros
  // above the diagonal included)
  if (t < RG_CB) {
    const int o = 16 * (t >> 4), j = t & 15;
    double x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double s0 = i == j ? 1.0 : 0.0, s1 = 0.0;
#pragma unroll
      for (int k = 0; k < i; ++k) {
        if (k & 1) s1 = fma(-Lu[(o + i) * RG_CS + o + k], x[k], s1);
        else s0 = fma(-Lu[(o + i) * RG_CS + o + k], x[k], s0);
      }
      x[i] = i >= j ? (s0 + s1) / Lu[(o + i) * RG_CS + o + i] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) X[(o + i) * RG_CS + o + j] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int h = 16; h < RG_CB; h *= 2) {  // blocks of size h combined into 2h
    const int npairs = RG_CB / (2 * h);
    // Tb = B A^-1 (B = L[o1 + r, o0 + k]; A^-1 is zero above its diagonal)
#pragma unroll
    for (int i = 0; i < npairs * h * h / 256; ++i) {
      const int e = t + 256 * i;
      const int pr = e / (h * h), r = (e / h) % h, c = e % h;
      const int o0 = 2 * h * pr, o1 = o0 + h;
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int k = 0; k < h; k += 2) {
        s0 = fma(Lu[(o1 + r) * RG_CS + o0 + k], X[(o0 + k) * RG_CS + o0 + c], s0);
        s1 = fma(Lu[(o1 + r) * RG_CS + o0 + k + 1], X[(o0 + k + 1) * RG_CS + o0 + c], s1);
      }
      Tb[e] = s0 + s1;
    }
    __syncthreads();
    // X[o1 + r, o0 + c] = -C^-1 Tb (C^-1 is zero above its diagonal)
#pragma unroll
    for (int i = 0; i < npairs * h * h / 256; ++i) {
      const int e = t + 256 * i;
      const int pr = e / (h * h), r = (e / h) % h, c = e % h;
      const int o0 = 2 * h * pr, o1 = o0 + h;
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int k = 0; k < h; k += 2) {
        s0 = fma(X[(o1 + r) * RG_CS + o1 + k], Tb[pr * h * h + k * h + c], s0);
        s1 = fma(X[(o1 + r) * RG_CS + o1 + k + 1], Tb[pr * h * h + (k + 1) * h + c], s1);
      }
      X[(o1 + r) * RG_CS + o0 + c] = -(s0 + s1);
    }
    __syncthreads();
  }
  for (int e = t; e < RG_CB * RG_CB; e += 256) {
    const int r = e / RG_CB, c = e % RG_CB;
    Li[e] = r >= c ? X[r * RG_CS + c] : 0.0;
  }
}

// Y[:, j] *= rs[j] over D rows of l columns (ld l).
__global__ __launch_bounds__(256) void rg_colscale_kernel(double* Y, int D, int l, const double* __restrict__ rs) {
  const size_t tot = (size_t)D * l;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) Y[e] *= rs[e % l];
}

// st[slot] = v.
__global__ void rg_set_kernel(int32_t* st, int slot, int v) { st[slot] = v; }

// Ritz order: rank the eigenvalues diag(S) (m of them) descending, ties by
// index; order[t] = index of rank t, sig[t] = sqrt(max(theta, 0)) for t < k.
// One workgroup.
__global__ __launch_bounds__(1024) void rg_order_kernel(const double* __restrict__ S, int ld, int m, int k,
                                                        int32_t* order, double* sig) {
  __shared__ double lam[1024];
  const int t = threadIdx.x;
  for (int i = t; i < m; i += blockDim.x) {
    const double v = S[(size_t)i * ld + i];
    lam[i] = isfinite(v) ? v : -INFINITY;
  }
  __syncthreads();
  for (int i = t; i < m; i += blockDim.x) {
    int rnk = 0;
    const double li = lam[i];
    for (int j = 0; j < m; ++j) rnk += (lam[j] > li) || (lam[j] == li && j < i);
    order[rnk] = i;
  }
  __syncthreads();
  for (int c = t; c < k; c += blockDim.x) sig[c] = sqrt(fmax(lam[order[c]], 0.0));
}

// W[:, c] = V[:, order[c]] for c < k (l rows).
__global__ __launch_bounds__(256) void rg_gather_kernel(const double* __restrict__ V, int ld, int l, int k,
                                                        const int32_t* __restrict__ order, double* W, int ldw) {
  const size_t tot = (size_t)l * k;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    const int r = (int)(e / k), c = (int)(e % k);
    W[(size_t)r * ldw + c] = V[(size_t)r * ld + order[c]];
  }
}

// B (fp32, D x R) and its bf16 copy from the fp64 basis Bk (D x k, ld k);
// columns k .. R-1 zero.
__global__ __launch_bounds__(256) void rg_store_basis_kernel(const double* __restrict__ Bk, int D, int k, int R,
                                                             float* B, uint16_t* Bbf) {
  const size_t tot = (size_t)D * R;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    const int d = (int)(e / R), c = (int)(e % R);
    const float v = c < k ? (float)Bk[(size_t)d * k + c] : 0.f;
    B[e] = v;
    Bbf[e] = iskv_to_bf16(v);
  }
}

// The refit's state: n rows, rank k, sigma = the Ritz singular values
// (zero past k), folded-row counter 0.
__global__ __launch_bounds__(256) void rg_commit_kernel(const double* __restrict__ sig, int k, int R, float* sigma,
                                                        int32_t* st, int n) {
  for (int c = threadIdx.x; c < R; c += 256) sigma[c] = c < k ? (float)sig[c] : 0.f;
  if (threadIdx.x == 0) {
    st[ST_N] = n;
    st[ST_K] = k;
    st[ST_FOLDED] = 0;
  }
}

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// Workspace of the Gram route: G (D x D), Y and V (D x l) in fp64, the Ritz
// singular values, the column scales, the Ritz order and the inverses of the
// Cholesky factor's 64 x 64 diagonal blocks.
size_t iskv_refit_gram_ws_bytes(const isvd_handle* h) {
  const size_t D = h->cfg.D, l = iskv_refit_block(h);
  const size_t P = (l + RG_CB - 1) / RG_CB;
  return al256(D * D * 8) + 2 * al256(D * l * 8) + 2 * al256(l * 8) + al256(l * 4) + al256(P * RG_CB * RG_CB * 8);
}

// Largest subspace block: r_max + b_max columns (the core eigensolver's
// order), at most D.
int iskv_refit_block(const isvd_handle* h) {
  const int l = h->m_max;
  return l < h->cfg.D ? l : h->cfg.D;
}

int iskv_launch_refit_gram(isvd_handle* h, const float* X, int32_t n, int32_t iters, void* work) {
  const iskv_config& c = h->cfg;
  isvd_ws& w = h->w;
  hipStream_t s = h->stream;
  const int D = c.D, R = c.r_max, ld = h->ldm;
  const int lmax = iskv_refit_block(h);
  // n rows span at most n directions: a block of n columns holds the whole
  // row space after the first step
  const int l = n < lmax ? n : lmax;
  int k = R < n ? R : n;
  if (k > D) k = D;
  char* wb = (char*)work;
  double* G = (double*)wb;
  double* Y = (double*)(wb + al256((size_t)D * D * 8));
  double* V = (double*)((char*)Y + al256((size_t)D * lmax * 8));
  double* sig = (double*)((char*)V + al256((size_t)D * lmax * 8));
  double* rs = (double*)((char*)sig + al256((size_t)lmax * 8));
  int32_t* order = (int32_t*)((char*)rs + al256((size_t)lmax * 8));
  double* Li = (double*)((char*)order + al256((size_t)lmax * 4));
  // 1. G = X^T X
  rg_gemm<true, false>(s, X, D, X, D, G, D, D, D, n, 1.0, 0.0);
  // orth(Y) -> V: CholeskyQR of the column-normalised Y with a relative
  // shift (two calls in a row: CholeskyQR2). Y is overwritten.
  const int P = (l + RG_CB - 1) / RG_CB;
  auto orth = [&](double* Yin, double* Vout, double rel) {
    double* Mm = w.Pa;   // Y^T Y (scaled), then its Cholesky factor (lower)
    rg_gemm<true, false>(s, (const double*)Yin, l, (const double*)Yin, l, Mm, ld, l, l, D, 1.0, 0.0, true);
    hipLaunchKernelGGL(rg_diag_kernel, dim3((l + 255) / 256), dim3(256), 0, s, (const double*)Mm, ld, l, rs);
    hipLaunchKernelGGL(rg_scale_kernel, dim3(128), dim3(256), 0, s, Mm, ld, l, (const double*)rs, rel);
    hipLaunchKernelGGL(rg_colscale_kernel, dim3(256), dim3(256), 0, s, Yin, D, l, (const double*)rs);
    for (int J = 0; J < P; ++J) {
      const int j0 = J * RG_CB, rest = l - j0 - RG_CB;
      double* LiJ = Li + (size_t)J * RG_CB * RG_CB;
      hipLaunchKernelGGL(rg_chol_diag_kernel, dim3(1), dim3(256), 0, s, Mm, ld, l, j0, rel, LiJ);
      if (rest > 0) {
        double* A21 = Mm + (size_t)(j0 + RG_CB) * ld + j0;
        double* A22 = A21 + RG_CB;
        // L21 = A21 L11^-T (in place), then A22 -= L21 L21^T (lower tiles)
        rg_gemm<false, true>(s, (const double*)A21, ld, (const double*)LiJ, RG_CB, A21, ld, rest, RG_CB, RG_CB, 1.0,
                             0.0);
        rg_gemm<false, true>(s, (const double*)A21, ld, (const double*)A21, ld, A22, ld, rest, rest, RG_CB, -1.0,
                             1.0, true);
      }
    }
    // V = Y L^-T by 64-column panels: V_J = (Y_J - V_<J L_J,<J^T) L_JJ^-T
    for (int J = 0; J < P; ++J) {
      const int j0 = J * RG_CB, nb = l - j0 < RG_CB ? l - j0 : RG_CB;
      const double* LiJ = Li + (size_t)J * RG_CB * RG_CB;
      if (J > 0)
        rg_gemm<false, true>(s, (const double*)Vout, l, (const double*)(Mm + (size_t)j0 * ld), ld, Yin + j0, l, D, nb,
                             j0, -1.0, 1.0);
      rg_gemm<false, true>(s, (const double*)(Yin + j0), l, LiJ, RG_CB, Vout + j0, l, D, nb, nb, 1.0, 0.0);
    }
  };
  // 2. random start, orthonormalised twice (CholeskyQR2; the buffers swap roles)
  hipLaunchKernelGGL(rg_rand_kernel, dim3(256), dim3(256), 0, s, Y, D, l);
  orth(Y, V, 1e-12);
  orth(V, Y, 1e-14);
  std::swap(V, Y);
  // 3. subspace iterations V <- orth(G V)
  for (int it = 0; it < iters; ++it) {
    rg_gemm<false, false>(s, (const double*)G, D, (const double*)V, l, Y, l, D, l, D, 1.0, 0.0);
    orth(Y, V, 1e-14);
  }
  // second pass on the last basis
  orth(V, Y, 1e-15);
  std::swap(V, Y);
  // 4. Rayleigh-Ritz: T = V^T (G V) into the core solver's matrix (dense: block Jacobi)
  rg_gemm<false, false>(s, (const double*)G, D, (const double*)V, l, Y, l, D, l, D, 1.0, 0.0);
  rg_gemm<true, false>(s, (const double*)V, l, (const double*)Y, l, w.A, ld, l, l, D, 1.0, 0.0);
  hipLaunchKernelGGL(rg_set_kernel, dim3(1), dim3(1), 0, s, w.st, (int)ST_JM, l);
  ISKV_HIP_CHECK(hipGetLastError());
  h->force_block_jacobi = true;
  int rc = iskv_launch_core_eig(h, ISKV_EIG_TOL_EXACT);
  h->force_block_jacobi = false;
  if (rc) return rc;
  hipLaunchKernelGGL(rg_order_kernel, dim3(1), dim3(1024), 0, s, (const double*)w.S, ld, l, k, order, sig);
  hipLaunchKernelGGL(rg_gather_kernel, dim3(128), dim3(256), 0, s, (const double*)w.V, ld, l, k,
                     (const int32_t*)order, w.W1, ld);
  // B = V W[:, :k] (D x k, into Y), stored fp32 + bf16
  rg_gemm<false, false>(s, (const double*)V, l, (const double*)w.W1, ld, Y, k, D, k, l, 1.0, 0.0);
  hipLaunchKernelGGL(rg_store_basis_kernel, dim3(256), dim3(256), 0, s, (const double*)Y, D, k, R, h->B, w.Bbf);
  hipLaunchKernelGGL(rg_commit_kernel, dim3(1), dim3(256), 0, s, (const double*)sig, k, R, h->sigma, w.st, n);
  ISKV_HIP_CHECK(hipGetLastError());
  // C = X B
  return iskv_launch_coords_from_rows(h, X, n);
}
