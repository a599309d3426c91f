// Block-incremental SVD merge and re-orthogonalisation on gfx950.
//
// Method: iS-KV notes (Zhou), §4.1-§4.4 and Algorithm 2. The history is kept
// as coordinates C = U diag(sigma) (n x k, fp32) and an orthonormal basis B
// (D x k, fp32). One merge of a pending block F (b x D):
//   Q = F B;  E = F - Q B^T;  E -= (E B) B^T            (projection, residual)
//   E E^T = V_E diag(rho^2) V_E^T, keep rho_j > tau      (residual basis)
//   P = E^T V_E[:, :p] diag(1/rho)                       (= P_E W of the notes)
//   M = [Q, F P];  Z^T Z = diag(sigma^2, 0) + M^T M      (core Gram, eq.(7))
//   Z^T Z = H diag(sigma+^2) H^T, keep r' = min(r, k+p)  (core SVD via Jacobi)
//   C_old <- C_old H[:k];  C_new = M H;  B <- [B, P] H   (coordinate sync)
// Storing C = U Sigma makes the old rows' update C H[:k] (= U G_top Sigma+)
// and the new rows M H (= G_bot Sigma+), so G is never formed and nothing is
// divided by a small singular value.
#include "iskv_internal.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

namespace {

// ----------------------------------------------------------------------------
// Device-side dimension: value = dev ? (*dev) * mul + add : v. Lets kernels be
// launched for the maximal shape while the actual extent (k, p, k+p, ...)
// lives in device memory, so a merge never waits for the host.
struct Dim {
  int v;
  const int32_t* dev;
  int mul;
  int add;
};
__device__ __forceinline__ int dval(const Dim& d) { return d.dev ? (*d.dev) * d.mul + d.add : d.v; }
static inline Dim hdim(int v) { return Dim{v, nullptr, 0, 0}; }
__device__ __forceinline__ void iskv_rb_dim(Dim& d, int64_t off) { d.dev = iskv_rb(d.dev, off); }
static inline Dim ddim(const int32_t* p, int mul = 1, int add = 0) { return Dim{0, p, mul, add}; }

// Ordering key of an eigenvalue: NaN sorts last as -inf, so that the rank
// "greater key, or equal key and lower index" is a strict total order and the
// ranks always form a permutation (a NaN must never leave a rank unassigned).
__device__ __forceinline__ double rank_key(double x) { return isnan(x) ? -INFINITY : x; }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values to packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32.
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
}

// ----------------------------------------------------------------------------
// Residual Gram E E^T in fp64 (b x b): workgroup (i, jb) forms row i against
// rows 8 jb .. 8 jb + 7, each thread over 4 consecutive features (D % 4 == 0),
// reduced over the wave and the 4 waves. Also latches the non-finite flag when
// the block (hence E) holds NaN or Inf.
__global__ __launch_bounds__(256) void resid_gram_kernel(const float* __restrict__ E, int D,
                                                         int b, double* GE, int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  E = iskv_rb(E, bdel);
  GE = iskv_rb(GE, bdel);
  st = iskv_rb(st, bdel);
  const int i = blockIdx.x, jb = blockIdx.y * 8;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double acc[8] = {};
  int bad = 0;
  for (int d = 4 * t; d < D; d += 1024) {
    const float4 x = *(const float4*)(E + (size_t)i * D + d);
    if (!(isfinite(x.x) && isfinite(x.y) && isfinite(x.z) && isfinite(x.w))) bad = 1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(jb + u, b - 1);
      const float4 y = *(const float4*)(E + (size_t)j * D + d);
      double a = acc[u];
      a = fma((double)x.x, (double)y.x, a);
      a = fma((double)x.y, (double)y.y, a);
      a = fma((double)x.z, (double)y.z, a);
      a = fma((double)x.w, (double)y.w, a);
      acc[u] = a;
    }
  }
  __shared__ double red[4][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    double v = acc[u];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) red[wave][u] = v;
  }
  __syncthreads();
  if (t < 8 && jb + t < b) GE[i * b + jb + t] = red[0][t] + red[1][t] + red[2][t] + red[3][t];
  if (bad && blockIdx.y == 0) atomicOr(&st[ST_STATUS], ISKV_DEV_NONFINITE);
}

// ----------------------------------------------------------------------------
// Residual basis (iS-KV notes §4.1): the residual directions of E^T with
// singular values rho_j above tau = max(delta s, max(D, b) 2^-23 s),
// s = max(sigma_1, rho_1), capped at p <= min(b, D - k). Published through
// V_E (b x b) and rho, so that P = E^T V_E diag(1/rho) (make_p_kernel).
//
// Both phases below diagonalise the b x b Gram E E^T (b <= 2 HB) by a
// parallel two-sided Jacobi in the systolic (Brent-Luk) arrangement: thread
// (I, J) of the HB x HB workgroup owns the 2 x 2 blocks at rows 2I, 2I+1 and
// columns 2J, 2J+1 of the working matrix S and of the eigenvector matrix V.
// Each round, every thread computes from the diagonal blocks the rotations of
// its pairs I and J (the symmetric 2 x 2 Schur rotation of Golub-Van Loan;
// each rotation is computed by every thread that needs it, from the same data,
// so all agree), applies S <- J_I^T S J_J and V <- V J_J to its blocks, and
// writes them to the positions of the next pairing of the round-robin
// (circle) schedule, so that 2 HB - 1 rounds pair every two indices once (one
// sweep). S and V are double-buffered in LDS: one barrier per round. The
// circle schedule moves every position through one cycle of length 2 HB - 1,
// so after each whole sweep every index is back at its own position. The Gram
// is zero-padded to 2 HB; padded indices never couple and are dropped.
//
// Phase 1 (when every residual direction can be kept, b <= D - k): sweeps in
// fp32 on S / trace until every scaled coupling |s_ij| / sqrt(s_ii s_jj) is
// below 3e-3, then S = V^T (E E^T) V is formed in fp64 from the fp32 V. If
// its couplings are below 1e-2 and Gershgorin's lower bound of its spectrum
// lies above tau^2 (tau from the upper bound of rho_1), then p = b and P only
// has to be an orthonormal basis of span(E^T), whose choice does not change
// the merge (the core changes by a rotation of its last b columns).
// P = E^T V S^-1/2 is one for any nonsingular V; S^-1/2 is taken as
// D^-1/2 (I - O/2 + 3 O^2 / 8) with D = diag(S), O = D^-1/2 S D^-1/2 - I
// (error 5/16 |O|^3 <= 3e-7, the fp32 rounding of P), so rho = 1, and the
// core block (F P)^T (F P) = S is diagonal up to couplings of 1e-2, which the
// core eigensolver resolves with the rest (rotations of that size among the
// new directions do not add a refinement step).
// Phase 2 (otherwise: a rank decision is needed, the residual is nearly
// degenerate, or phase 1 did not certify): fp64 sweeps from the Gram until
// none rotates; an off-diagonal is rotated away when it exceeds 1e-13 of the
// geometric mean of its diagonal pair and 1e-15 of the trace. Eigenvalues are
// ranked and thresholded exactly.
// Round-robin move of position x: pairs are (2k, 2k+1); position 0 stays, the
// others cycle 1 -> 2 -> 4 -> ... -> 2h-2 -> 2h-1 -> 2h-3 -> ... -> 3 -> 1.
__device__ __forceinline__ int rr_next(int x, int h) {
  if (x == 0) return 0;
  if (x == 1) return 2;
  if ((x & 1) == 0) return x == 2 * (h - 1) ? x + 1 : x + 2;
  return x - 2;
}

// fp64 rotation [[c, s], [-s, c]] with J^T [[app, apq], [apq, aqq]] J (nearly)
// diagonal. With d = aqq - app, r = sqrt(d^2 + 4 apq^2) and w = |d| + r, the
// annihilating rotation has c = w / sqrt(2 r w), s = sign(d) 2 apq / sqrt(2 r w).
// The angle is computed in fp32 on the inputs scaled by 1/trace (so they lie
// in [1e-15, 1]); (c, s) is then normalised in fp64 by two Newton steps for
// 1/sqrt(c^2 + s^2), so the rotation is orthogonal to fp64 precision. It
// leaves an off-diagonal of about 1e-7 of the old one, which later sweeps
// remove. Below threshold the identity is returned (selected after the
// arithmetic: no branch).
__device__ __forceinline__ bool schur2(double app, double apq, double aqq, double abs_tol, double inv_tr,
                                       double& c, double& sn) {
  const bool rot = fabs(apq) > abs_tol && apq * apq > 1e-26 * fabs(app * aqq);
  const float p = (float)(app * inv_tr), q = (float)(aqq * inv_tr), o = (float)(apq * inv_tr);
  const float d = q - p;
  const float r = __fsqrt_rn(fmaf(d, d, 4.0f * o * o));
  const float w = fabsf(d) + r;
  const float rq = __frsqrt_rn(2.0f * r * w);
  const double c0 = (double)(w * rq);
  const double s0 = (double)((d >= 0.0f ? 2.0f : -2.0f) * o * rq);
  const double n2 = c0 * c0 + s0 * s0;
  double y = 1.5 - 0.5 * n2;
  y = y * (1.5 - 0.5 * n2 * y * y);
  c = rot ? c0 * y : 1.0;
  sn = rot ? s0 * y : 0.0;
  return rot;
}

// The same rotation in fp32 for phase 1 (orthogonal to fp32 precision, which
// phase 1 does not need: V only has to be nonsingular). Rotates when the
// scaled coupling exceeds 1e-5.
__device__ __forceinline__ bool schur2f(float app, float apq, float aqq, float& c, float& sn) {
  const bool rot = apq * apq > 1e-10f * fabsf(app * aqq) && apq != 0.0f;
  const float d = aqq - app;
  const float r = __builtin_amdgcn_sqrtf(fmaf(d, d, 4.0f * apq * apq));
  const float w = fabsf(d) + r;
  const float rq = __frsqrt_rn(2.0f * r * w);
  c = rot ? w * rq : 1.0f;
  sn = rot ? (d >= 0.0f ? 2.0f : -2.0f) * apq * rq : 0.0f;
  return rot;
}

constexpr int RB32_MAX_SWEEPS = 12;

// LDS layout (dynamic): phase 1 uses fp32 S[2][N][LF], V[2][N][LF] at the
// start and fp64 G[N][L], T[N][L] after them; phase 2 reuses the start for
// fp64 S[2][N][L], V[2][N][L]. LF = N + 16 for N = 32 puts the two rows a
// 64-lane read touches on opposite halves of the banks; for N = 64 one row
// fills a half-wave.
template <int HB> constexpr int rb_lf() { return HB == 16 ? 48 : 2 * HB + 2; }
static inline size_t resid_lds_bytes(int hb) {
  const size_t n = 2 * hb, l = n + 1, lf = hb == 16 ? 48 : n + 2;
  const size_t p1 = 4 * n * lf * sizeof(float) + 2 * n * l * sizeof(double);
  const size_t p2 = 4 * n * l * sizeof(double);
  return p1 > p2 ? p1 : p2;
}

template <int HB>
__global__ __launch_bounds__(HB * HB) void resid_basis_kernel(const double* __restrict__ GE, int b,
                                                              int D, const float* __restrict__ sigma,
                                                              float delta, double* VE, double* rho,
                                                              int32_t* st, int max_sweeps,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  GE = iskv_rb(GE, bdel);
  sigma = iskv_rb(sigma, bdel);
  VE = iskv_rb(VE, bdel);
  rho = iskv_rb(rho, bdel);
  st = iskv_rb(st, bdel);
  constexpr int N = 2 * HB, L = N + 1, LF = rb_lf<HB>();
  constexpr int NW = HB * HB / 64;
  extern __shared__ double rb_lds[];
  __shared__ double lam[N];
  __shared__ int order[N];
  __shared__ double wred[3][NW];
  const int t = threadIdx.x, I = t / HB, J = t % HB;
  const int r0 = 2 * I, r1 = r0 + 1, c0 = 2 * J, c1 = c0 + 1;
  const int pr0 = rr_next(r0, HB), pr1 = rr_next(r1, HB), pc0 = rr_next(c0, HB), pc1 = rr_next(c1, HB);
  auto g = [&](int i, int j) { return (i < b && j < b) ? GE[i * b + j] : 0.0; };
  const double g11 = g(r0, c0), g12 = g(r0, c1), g21 = g(r1, c0), g22 = g(r1, c1);
  const int nonzero = __syncthreads_or(g11 != 0.0 || g12 != 0.0 || g21 != 0.0 || g22 != 0.0);
  const int k = st[ST_K];
  if (!nonzero || k >= D) {
    if (t == 0) { st[ST_P] = 0; st[ST_M] = k; st[ST_EZERO] = nonzero ? 0 : 1; }
    return;
  }
  if (I == J) { lam[r0] = g11; lam[r1] = g22; }
  __syncthreads();
  double trace = 0.0;
  for (int i = 0; i < N; ++i) trace += fabs(lam[i]);
  const double inv_tr = 1.0 / trace;
  const double s1 = (k > 0) ? (double)sigma[0] : 0.0;
  const double tfac = fmax((double)delta, (double)(D > b ? D : b) * 1.1920928955078125e-07);
  int sweeps = 0;
  __syncthreads();  // lam is rewritten below

  // ---------------------------------------------------------------- phase 1
  if (b <= D - k) {
    float* Sf = (float*)rb_lds;  // [2][N][LF]
    float* Vf = Sf + 2 * N * LF;  // [2][N][LF]
    double* G64 = rb_lds + 2 * N * LF;  // [N][L] (after the fp32 buffers)
    double* T64 = G64 + N * L;          // [N][L]
    {
      const float f = (float)inv_tr;
      Sf[r0 * LF + c0] = (float)g11 * f; Sf[r0 * LF + c1] = (float)g12 * f;
      Sf[r1 * LF + c0] = (float)g21 * f; Sf[r1 * LF + c1] = (float)g22 * f;
      Vf[r0 * LF + c0] = r0 == c0; Vf[r0 * LF + c1] = 0.0f; Vf[r1 * LF + c0] = 0.0f; Vf[r1 * LF + c1] = r1 == c1;
      G64[r0 * L + c0] = g11; G64[r0 * L + c1] = g12; G64[r1 * L + c0] = g21; G64[r1 * L + c1] = g22;
    }
    __syncthreads();
    int cur = 0;
    for (int sweep = 0; sweep < RB32_MAX_SWEEPS; ++sweep) {
      ++sweeps;
      int rotated = 0;
      for (int round = 0; round < N - 1; ++round) {
        const float* S = Sf + cur * N * LF;
        const float* V = Vf + cur * N * LF;
        const float ap = S[r0 * LF + r0], apq = S[r0 * LF + r1], aq = S[r1 * LF + r1];
        const float bp = S[c0 * LF + c0], bpq = S[c0 * LF + c1], bq = S[c1 * LF + c1];
        float x11 = S[r0 * LF + c0], x12 = S[r0 * LF + c1], x21 = S[r1 * LF + c0], x22 = S[r1 * LF + c1];
        float v11 = V[r0 * LF + c0], v12 = V[r0 * LF + c1], v21 = V[r1 * LF + c0], v22 = V[r1 * LF + c1];
        float ca, sa, cb, sb;
        rotated |= schur2f(ap, apq, aq, ca, sa);
        schur2f(bp, bpq, bq, cb, sb);
        {
          const float y11 = ca * x11 - sa * x21, y12 = ca * x12 - sa * x22;
          const float y21 = sa * x11 + ca * x21, y22 = sa * x12 + ca * x22;
          x11 = y11 * cb - y12 * sb; x12 = y11 * sb + y12 * cb;
          x21 = y21 * cb - y22 * sb; x22 = y21 * sb + y22 * cb;
        }
        if (I == J) {
          const float m = 0.5f * (x12 + x21);
          x12 = m; x21 = m;
        }
        {
          const float w11 = v11 * cb - v12 * sb, w12 = v11 * sb + v12 * cb;
          const float w21 = v21 * cb - v22 * sb, w22 = v21 * sb + v22 * cb;
          v11 = w11; v12 = w12; v21 = w21; v22 = w22;
        }
        cur ^= 1;
        float* So = Sf + cur * N * LF;
        float* Vo = Vf + cur * N * LF;
        So[pr0 * LF + pc0] = x11; So[pr0 * LF + pc1] = x12; So[pr1 * LF + pc0] = x21; So[pr1 * LF + pc1] = x22;
        Vo[r0 * LF + pc0] = v11; Vo[r0 * LF + pc1] = v12; Vo[r1 * LF + pc0] = v21; Vo[r1 * LF + pc1] = v22;
        __syncthreads();
      }
      if (!__syncthreads_or(rotated)) break;
      if (sweep >= 1) {  // largest scaled coupling left
        const float* S = Sf + cur * N * LF;
        auto cpl = [&](int i, int j) {
          return (i != j && i < b && j < b)
                     ? fabsf(S[i * LF + j]) / sqrtf(fabsf(S[i * LF + i] * S[j * LF + j]) + 1e-37f) : 0.0f;
        };
        float om = fmaxf(fmaxf(cpl(r0, c0), cpl(r0, c1)), fmaxf(cpl(r1, c0), cpl(r1, c1)));
        if (__syncthreads_and(!(om >= 3e-3f))) break;  // NaN stays in the loop, fails below
      }
    }
    const float* Vc = Vf + cur * N * LF;
    // T = G V (fp64), then this thread's block of S = V^T T
    {
      double t11 = 0.0, t12 = 0.0, t21 = 0.0, t22 = 0.0;
      for (int a = 0; a < N; ++a) {
        const double ga0 = G64[r0 * L + a], ga1 = G64[r1 * L + a];
        const double va0 = Vc[a * LF + c0], va1 = Vc[a * LF + c1];
        t11 = fma(ga0, va0, t11); t12 = fma(ga0, va1, t12);
        t21 = fma(ga1, va0, t21); t22 = fma(ga1, va1, t22);
      }
      T64[r0 * L + c0] = t11; T64[r0 * L + c1] = t12; T64[r1 * L + c0] = t21; T64[r1 * L + c1] = t22;
    }
    __syncthreads();
    double y11 = 0.0, y12 = 0.0, y21 = 0.0, y22 = 0.0;
    for (int a = 0; a < N; ++a) {
      const double va0 = Vc[a * LF + r0], va1 = Vc[a * LF + r1];
      const double ta0 = T64[a * L + c0], ta1 = T64[a * L + c1];
      y11 = fma(va0, ta0, y11); y12 = fma(va0, ta1, y12);
      y21 = fma(va1, ta0, y21); y22 = fma(va1, ta1, y22);
    }
    if (I == J) { lam[r0] = y11; lam[r1] = y22; }
    __syncthreads();
    const bool q0 = r0 < b, q1 = r1 < b, p0 = c0 < b, p1 = c1 < b;
    const double d0 = lam[r0], d1 = lam[r1], e0 = lam[c0], e1 = lam[c1];
    auto relo = [&](double v, double da, double db, bool ra, bool cb, bool diag) {
      return (ra && cb && !diag) ? fabs(v) / sqrt(fabs(da * db)) : 0.0;
    };
    double offm = fmax(fmax(relo(y11, d0, e0, q0, p0, r0 == c0), relo(y12, d0, e1, q0, p1, r0 == c1)),
                       fmax(relo(y21, d1, e0, q1, p0, r1 == c0), relo(y22, d1, e1, q1, p1, r1 == c1)));
    double rs0 = ((p0 && c0 != r0) ? fabs(y11) : 0.0) + ((p1 && c1 != r0) ? fabs(y12) : 0.0);
    double rs1 = ((p0 && c0 != r1) ? fabs(y21) : 0.0) + ((p1 && c1 != r1) ? fabs(y22) : 0.0);
#pragma unroll
    for (int o = 1; o < HB; o <<= 1) {
      rs0 += __shfl_xor(rs0, o, 64);
      rs1 += __shfl_xor(rs1, o, 64);
    }
    double lo = INFINITY, hi = 0.0;
    if (J == 0) {
      if (q0) { lo = fmin(lo, d0 - rs0); hi = fmax(hi, d0 + rs0); }
      if (q1) { lo = fmin(lo, d1 - rs1); hi = fmax(hi, d1 + rs1); }
    }
    if (isnan(offm)) offm = INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      offm = fmax(offm, __shfl_xor(offm, o, 64));
      lo = fmin(lo, __shfl_xor(lo, o, 64));
      hi = fmax(hi, __shfl_xor(hi, o, 64));
    }
    if ((t & 63) == 0) { wred[0][t >> 6] = offm; wred[1][t >> 6] = lo; wred[2][t >> 6] = hi; }
    __syncthreads();
    double om = 0.0, lm = INFINITY, hm = 0.0;
    for (int w = 0; w < NW; ++w) {
      om = fmax(om, wred[0][w]);
      lm = fmin(lm, wred[1][w]);
      hm = fmax(hm, wred[2][w]);
    }
    const double tau_hi = tfac * fmax(s1, sqrt(hm));
    if (om < 1e-2 && lm > tau_hi * tau_hi) {  // same decision in every thread
      // O = D^-1/2 S D^-1/2 - I over the real indices (into G64's place),
      // Z = D^-1/2 (I - O/2 + 3 O^2 / 8) (into T64's place), V_E = V Z.
      double* Ob = G64;
      double* Zb = T64;
      const double sr0 = q0 ? 1.0 / sqrt(d0) : 0.0, sr1 = q1 ? 1.0 / sqrt(d1) : 0.0;
      const double sc0 = p0 ? 1.0 / sqrt(e0) : 0.0, sc1 = p1 ? 1.0 / sqrt(e1) : 0.0;
      const double o11 = r0 == c0 ? 0.0 : y11 * sr0 * sc0, o12 = r0 == c1 ? 0.0 : y12 * sr0 * sc1;
      const double o21 = r1 == c0 ? 0.0 : y21 * sr1 * sc0, o22 = r1 == c1 ? 0.0 : y22 * sr1 * sc1;
      Ob[r0 * L + c0] = o11; Ob[r0 * L + c1] = o12; Ob[r1 * L + c0] = o21; Ob[r1 * L + c1] = o22;
      __syncthreads();
      double q11 = 0.0, q12 = 0.0, q21 = 0.0, q22 = 0.0;
      for (int x = 0; x < N; ++x) {
        const double a0 = Ob[r0 * L + x], a1 = Ob[r1 * L + x], b0 = Ob[x * L + c0], b1 = Ob[x * L + c1];
        q11 = fma(a0, b0, q11); q12 = fma(a0, b1, q12); q21 = fma(a1, b0, q21); q22 = fma(a1, b1, q22);
      }
      auto zv = [&](int r, int c, double o, double o2, double sr) {
        return sr * ((r == c ? 1.0 : 0.0) - 0.5 * o + 0.375 * o2);
      };
      Zb[r0 * L + c0] = zv(r0, c0, o11, q11, sr0);
      Zb[r0 * L + c1] = zv(r0, c1, o12, q12, sr0);
      Zb[r1 * L + c0] = zv(r1, c0, o21, q21, sr1);
      Zb[r1 * L + c1] = zv(r1, c1, o22, q22, sr1);
      __syncthreads();
      for (int idx = t; idx < b * b; idx += HB * HB) {
        const int row = idx / b, j = idx % b;
        double acc = 0.0;
        for (int x = 0; x < N; ++x) acc = fma((double)Vc[row * LF + x], Zb[x * L + j], acc);
        VE[row * b + j] = acc;
      }
      if (t < b) rho[t] = 1.0;
      if (t == 0) { st[ST_P] = b; st[ST_M] = k + b; st[ST_EZERO] = 0; st[ST_RSWEEPS] = sweeps; }
      return;
    }
    __syncthreads();  // phase 2 reuses the LDS
  }

  // ---------------------------------------------------------------- phase 2
  double* Sb = rb_lds;              // [2][N][L]
  double* Vb = rb_lds + 2 * N * L;  // [2][N][L]
  double x11 = g11, x12 = g12, x21 = g21, x22 = g22;
  Sb[r0 * L + c0] = x11; Sb[r0 * L + c1] = x12; Sb[r1 * L + c0] = x21; Sb[r1 * L + c1] = x22;
  Vb[r0 * L + c0] = r0 == c0; Vb[r0 * L + c1] = 0.0; Vb[r1 * L + c0] = 0.0; Vb[r1 * L + c1] = r1 == c1;
  __syncthreads();
  const double abs_tol = 1e-15 * trace;
  int cur = 0;
  for (int sweep = 0; sweep < max_sweeps; ++sweep) {
    ++sweeps;
    int rotated = 0;
    for (int round = 0; round < N - 1; ++round) {
      const double* S = Sb + cur * N * L;
      const double* V = Vb + cur * N * L;
      // every LDS value of the round is read up front
      const double ap = S[r0 * L + r0], apq = S[r0 * L + r1], aq = S[r1 * L + r1];
      const double bp = S[c0 * L + c0], bpq = S[c0 * L + c1], bq = S[c1 * L + c1];
      x11 = S[r0 * L + c0]; x12 = S[r0 * L + c1]; x21 = S[r1 * L + c0]; x22 = S[r1 * L + c1];
      double v11 = V[r0 * L + c0], v12 = V[r0 * L + c1], v21 = V[r1 * L + c0], v22 = V[r1 * L + c1];
      double ca, sa, cb, sb;
      rotated |= schur2(ap, apq, aq, abs_tol, inv_tr, ca, sa);
      schur2(bp, bpq, bq, abs_tol, inv_tr, cb, sb);
      {  // S <- J_I^T S J_J on this block
        const double y11 = ca * x11 - sa * x21, y12 = ca * x12 - sa * x22;
        const double y21 = sa * x11 + ca * x21, y22 = sa * x12 + ca * x22;
        x11 = y11 * cb - y12 * sb; x12 = y11 * sb + y12 * cb;
        x21 = y21 * cb - y22 * sb; x22 = y21 * sb + y22 * cb;
      }
      if (I == J) {  // keep the diagonal blocks exactly symmetric
        const double m = 0.5 * (x12 + x21);
        x12 = m; x21 = m;
      }
      {  // V <- V J_J
        const double w11 = v11 * cb - v12 * sb, w12 = v11 * sb + v12 * cb;
        const double w21 = v21 * cb - v22 * sb, w22 = v21 * sb + v22 * cb;
        v11 = w11; v12 = w12; v21 = w21; v22 = w22;
      }
      // next pairing: S'[pi(i)][pi(j)] = S[i][j], V'[i][pi(j)] = V[i][j]
      cur ^= 1;
      double* So = Sb + cur * N * L;
      double* Vo = Vb + cur * N * L;
      So[pr0 * L + pc0] = x11; So[pr0 * L + pc1] = x12; So[pr1 * L + pc0] = x21; So[pr1 * L + pc1] = x22;
      Vo[r0 * L + pc0] = v11; Vo[r0 * L + pc1] = v12; Vo[r1 * L + pc0] = v21; Vo[r1 * L + pc1] = v22;
      __syncthreads();
    }
    if (!__syncthreads_or(rotated)) break;
  }
  // whole sweeps only: original index j sits at position j
  const double* S = Sb + cur * N * L;
  const double* V = Vb + cur * N * L;
  if (t == 0) st[ST_RSWEEPS] = sweeps;
  if (t < b) lam[t] = S[t * L + t];
  __syncthreads();
  // rank by descending eigenvalue, ties by index (NaN last)
  if (t < b) {
    int rnk = 0;
    const double ki = rank_key(lam[t]);
    for (int j = 0; j < b; ++j) {
      const double kj = rank_key(lam[j]);
      rnk += (kj > ki) || (kj == ki && j < t);
    }
    order[rnk] = t;
  }
  __syncthreads();
  for (int idx = t; idx < b * b; idx += HB * HB) {
    const int row = idx / b, col = idx % b;
    VE[row * b + col] = V[row * L + min(max(order[col], 0), b - 1)];
  }
  if (t < b) rho[t] = sqrt(fmax(lam[min(max(order[t], 0), b - 1)], 0.0));
  if (t == 0) {
    const double rho1 = sqrt(fmax(lam[min(max(order[0], 0), b - 1)], 0.0));
    const double tau = tfac * fmax(s1, rho1);
    int p = 0;
    for (int j = 0; j < b; ++j) p += sqrt(fmax(lam[min(max(order[j], 0), b - 1)], 0.0)) > tau;
    if (p > D - k) p = D - k;
    st[ST_P] = p;
    st[ST_M] = k + p;
    st[ST_EZERO] = 0;
  }
}

// P[:, j] = E^T V_E[:, j] / rho_j for j < p (D x b_max, fp64 accumulation).
// Workgroup: 64 features d and all columns; thread (d, g) forms columns
// 8 g .. 8 g + 7 of row d from V_E staged in LDS (the rows of E are read
// coalesced along d, all b of them in flight at once) and writes them as
// 32 contiguous bytes.
constexpr int MP_BMAX = 64;  // largest block (b_max <= 64: at most 512 threads, 33 KiB of LDS)
__global__ __launch_bounds__(8 * MP_BMAX) void make_p_kernel(const float* __restrict__ E, int D, int b,
                                                      const double* __restrict__ VE,
                                                      const double* __restrict__ rho, float* P,
                                                      int ldp, const int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  E = iskv_rb(E, bdel);
  VE = iskv_rb(VE, bdel);
  rho = iskv_rb(rho, bdel);
  P = iskv_rb(P, bdel);
  st = iskv_rb(st, bdel);
  extern __shared__ double mp_lds[];  // V_E (b x b), then 1 / rho (b)
  const int p = st[ST_P];
  const int t = threadIdx.x, d = blockIdx.x * 64 + (t & 63), g = t >> 6;
  for (int e = t; e < b * b; e += blockDim.x) mp_lds[e] = VE[e];
  for (int e = t; e < b; e += blockDim.x) mp_lds[b * b + e] = e < p ? 1.0 / rho[e] : 0.0;
  __syncthreads();
  if (d >= D || 8 * g >= p) return;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int i0 = 0; i0 < b; i0 += 16) {
    float ev[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) ev[u] = E[(size_t)min(i0 + u, b - 1) * D + d];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (i0 + u < b) {
        const double x = (double)ev[u];
        const double* v = mp_lds + (i0 + u) * b;
        // columns past b are never stored: their index is only kept in range
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fma(x, v[min(8 * g + q, b - 1)], acc[q]);
      }
    }
  }
  float o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = (float)(acc[q] * mp_lds[b * b + min(8 * g + q, b - 1)]);
  float* dst = P + (size_t)d * ldp + 8 * g;
  if (8 * g + 8 <= p && (ldp & 3) == 0) {
    *(float4*)dst = float4{o[0], o[1], o[2], o[3]};
    *(float4*)(dst + 4) = float4{o[4], o[5], o[6], o[7]};
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (8 * g + q < p) dst[q] = o[q];
  }
}

// Core Gram A = diag(sigma^2, 0_p) + M^T M in fp64, M = [Q[:, :k], FP[:, :p]] (b x m);
// also sets ST_JM = m for the eigensolver.
__global__ __launch_bounds__(256) void core_gram_kernel(const float* __restrict__ Q, int ldq,
                                                        const float* __restrict__ FP, int ldfp,
                                                        const float* __restrict__ sigma, int b,
                                                        double* A, int lda, int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  Q = iskv_rb(Q, bdel);
  FP = iskv_rb(FP, bdel);
  sigma = iskv_rb(sigma, bdel);
  A = iskv_rb(A, bdel);
  st = iskv_rb(st, bdel);
  const int k = st[ST_K], m = st[ST_M];
  // the eigensolver's order (no other workgroup of this launch reads it)
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) st[ST_JM] = m;
  const int i = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int j = blockIdx.x * 16 + (threadIdx.x & 15);
  if (i >= m || j >= m) return;
  // column i (j) of M = [Q[:, :k], FP[:, :p]]: base and row stride
  const float* pi = i < k ? Q + i : FP + (i - k);
  const float* pj = j < k ? Q + j : FP + (j - k);
  const int si = i < k ? ldq : ldfp, sj = j < k ? ldq : ldfp;
  double acc = 0.0;
  for (int r0 = 0; r0 < b; r0 += 8) {  // 8 rows' loads in flight before their products
    float mi[8], mj[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = min(r0 + u, b - 1);
      mi[u] = pi[(size_t)r * si];
      mj[u] = pj[(size_t)r * sj];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r0 + u < b) acc = fma((double)mi[u], (double)mj[u], acc);
  }
  if (i == j && i < k) acc += (double)sigma[i] * (double)sigma[i];
  A[(size_t)i * lda + j] = acc;
}

// Sort eigenpairs by descending eigenvalue, keep `keep` of them:
// order[t] (rank order), sig_new[t] = sqrt(max(lambda, 0)), ST_KNEW = keep.
// keep = min(r_max, n) for a merge; n for re-orthogonalisation. One workgroup.
__global__ __launch_bounds__(1024) void eig_order_kernel(const double* __restrict__ S, int ld,
                                                         float* sig_new, int32_t* order, int32_t* st,
                                                         int r_max, int for_merge,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  S = iskv_rb(S, bdel);
  sig_new = iskv_rb(sig_new, bdel);
  order = iskv_rb(order, bdel);
  st = iskv_rb(st, bdel);
  __shared__ double lam[1024], key[1024];
  __shared__ int rnk[1024], ord[1024];
  const int n = st[ST_JM];
  const int t = threadIdx.x;
  for (int i = t; i < n; i += blockDim.x) {
    lam[i] = S[(size_t)i * ld + i];
    key[i] = rank_key(lam[i]);
    rnk[i] = 0;
  }
  __syncthreads();
  // rank of i = entries ahead of it (larger, or equal at a lower index); the
  // n x n comparisons are split over the workgroup in quarters of j, read
  // eight keys at a time
  const int qn = (n + 3) / 4;
  for (int e = t; e < 4 * n; e += blockDim.x) {
    const int i = e >> 2, j0 = (e & 3) * qn, j1 = min(j0 + qn, n);
    const double ki = key[i];
    int c = 0;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
      double kj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kj[u] = key[j + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) c += (kj[u] > ki) || (kj[u] == ki && j + u < i);
    }
    for (; j < j1; ++j) {
      const double kj = key[j];
      c += (kj > ki) || (kj == ki && j < i);
    }
    atomicAdd(&rnk[i], c);
  }
  __syncthreads();
  for (int i = t; i < n; i += blockDim.x) ord[rnk[i]] = i;
  __syncthreads();
  for (int i = t; i < n; i += blockDim.x) order[i] = ord[i];
  const int keep = for_merge ? (n < r_max ? n : r_max) : n;
  for (int c = t; c < keep; c += blockDim.x) sig_new[c] = (float)sqrt(fmax(lam[min(max(ord[c], 0), n - 1)], 0.0));
  if (t == 0 && for_merge) st[ST_KNEW] = keep;
}

// Hc[:, t] = V[:, order[t]] (fp32, ld r_max) for the kept columns. A kept
// column whose index is an old direction (t < k) is signed so that
// H[t, t] >= 0, i.e. the basis moves continuously; the synced product does
// not depend on it, the basis-only ablation does. Grid-stride, many blocks.
// With Hf, also writes H in the operand order of xh_reg_kernel (XF_KQ groups
// of four k steps per wave): element j of float4 ((w XF_KQ + q) 64 + l) is
// H[4 (4 q + j) + l / 16, 16 w + l % 16] (zero outside n x keep), so each lane
// of the right-multiplication loads its H operands as 16-byte pieces.
constexpr int XF_KQ = 18;  // 72 k steps of 4: rows up to 288
__global__ __launch_bounds__(256) void eig_gather_kernel(const double* __restrict__ V, int ld,
                                                         float* Hc, int ldh,
                                                         const int32_t* __restrict__ order,
                                                         const int32_t* __restrict__ st, int r_max,
                                                         int for_merge, float* Hf,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  V = iskv_rb(V, bdel);
  Hc = iskv_rb(Hc, bdel);
  order = iskv_rb(order, bdel);
  st = iskv_rb(st, bdel);
  Hf = iskv_rb(Hf, bdel);
  const int n = st[ST_JM];
  const int keep = for_merge ? (n < r_max ? n : r_max) : n;
  const int kold = for_merge ? st[ST_K] : 0;
  const size_t tot = (size_t)n * keep;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int row = (int)(e / keep), col = (int)(e % keep);
    const int oc = min(max(order[col], 0), n - 1);
    double v = V[(size_t)row * ld + oc];
    if (col < kold && V[(size_t)col * ld + oc] < 0.0) v = -v;
    Hc[(size_t)row * ldh + col] = (float)v;
  }
  if (Hf) {
    constexpr int NF = 16 * XF_KQ * 64 * 4;
    for (int e = blockIdx.x * 256 + threadIdx.x; e < NF; e += gridDim.x * 256) {
      const int j = e & 3, l = (e >> 2) & 63, q = (e >> 8) % XF_KQ, w = (e >> 8) / XF_KQ;
      const int row = 4 * (4 * q + j) + (l >> 4), col = 16 * w + (l & 15);
      double v = 0.0;
      if (row < n && col < keep) {
        const int oc = min(max(order[col], 0), n - 1);
        v = V[(size_t)row * ld + oc];
        if (col < kold && V[(size_t)col * ld + oc] < 0.0) v = -v;
      }
      Hf[e] = (float)v;
    }
  }
}

// ----------------------------------------------------------------------------
// Right-multiplication by a small matrix on fp32 MFMA (v_mfma_f32_16x16x4f32):
//   Y[i, :kout] = X[i, :kin] H[:kin, :kout],   X = [X1[:, :k1] | X2[:, :kin-k1]].
// Serves the coordinate update C <- C H (in place), the basis update
// B <- [B | P] H (in place, with the bf16 copy) and the new rows
// [Q | F P] H. A workgroup owns BM (16 or 32) rows: it stages all kin columns
// of its rows in LDS before writing any output, so in-place use is safe
// (workgroups own disjoint rows). H streams through LDS in 32-deep chunks,
// the next chunk's loads in flight while the current one is multiplied.
// Output columns go in tiles of 256; wave w owns 16-column blocks 4w .. 4w+3.
typedef float v4f_t __attribute__((ext_vector_type(4)));
constexpr int XH_KC = 32;             // H chunk depth
constexpr int XH_NT = 256;            // output column tile
constexpr int XH_HS = XH_NT + 16;     // LDS row stride of the H chunk (floats)

__host__ __device__ inline int xh_ldx(int kin_max) { return (kin_max + 7) / 8 * 8 + 4; }
static inline size_t xh_lds_bytes(int bm, int kin_max) {
  return ((size_t)bm * xh_ldx(kin_max) + (size_t)XH_KC * XH_HS) * sizeof(float);
}

template <int BM, typename TX, typename TY>
__global__ __launch_bounds__(256) void xh_mfma_kernel(const TX* X1, int ld1, const float* X2, int ld2,
                                                      Dim k1_d, Dim kin_d, const float* __restrict__ H,
                                                      int ldh, int hcols, Dim kout_d, Dim rows_d,
                                                      TY* Y, int ldy, uint16_t* Ybf, int ldbf,
                                                      int ldx, int32_t* pos, const int32_t* pos_src,
                                                      Dim yoff_d, int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X1 = iskv_rb(X1, bdel);
  X2 = iskv_rb(X2, bdel);
  iskv_rb_dim(k1_d, bdel);
  iskv_rb_dim(kin_d, bdel);
  H = iskv_rb(H, bdel);
  iskv_rb_dim(kout_d, bdel);
  iskv_rb_dim(rows_d, bdel);
  Y = iskv_rb(Y, bdel);
  Ybf = iskv_rb(Ybf, bdel);
  pos = iskv_rb(pos, bdel);
  pos_src = iskv_rb(pos_src, bdel);
  st = iskv_rb(st, bdel);
  iskv_rb_dim(yoff_d, bdel);
  const int k1 = dval(k1_d), kin = dval(kin_d), kout = dval(kout_d), rows = dval(rows_d);
  const int yo = dval(yoff_d);
  const int i0 = blockIdx.x * BM;
  if (i0 >= rows || kout <= 0) return;
  extern __shared__ float sm[];
  float* Xs = sm;               // [BM][ldx]
  float* Hs = sm + BM * ldx;    // [XH_KC][XH_HS]
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nr = min(BM, rows - i0);
  bool over = false;  // a saturated half store (fp16 coordinates only)
  // X tile: all loads issued, then stored; zero beyond kin and nr
  {
    const int kin4 = (kin + 3) & ~3;
    for (int base = 0; base < BM * kin4; base += 256 * 16) {
      float xv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int e = base + t + 256 * u, r = e / kin4, c = e - r * kin4;
        int rc = min(r, nr - 1);
        float v = 0.f;
        if (e < BM * kin4 && c < kin)
          v = c < k1 ? iskv_ld(X1 + (size_t)(i0 + rc) * ld1 + c) : X2[(size_t)(i0 + rc) * ld2 + (c - k1)];
        xv[u] = (r < nr) ? v : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        int e = base + t + 256 * u, r = e / kin4, c = e - r * kin4;
        if (e < BM * kin4) Xs[r * ldx + c] = xv[u];
      }
    }
  }
  if (pos && t < nr) pos[yo + i0 + t] = pos_src[t + i0];
  constexpr int RB = BM / 16;
  const int nch = (kin + XH_KC - 1) / XH_KC;
  for (int j0 = 0; j0 < kout; j0 += XH_NT) {
    v4f_t acc[RB][4];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = v4f_t{0.f, 0.f, 0.f, 0.f};
    // H chunk element (kk, jj): e = t + 256 u, kk = e / 256, jj = e % 256
    float hr[XH_KC];
    auto load_h = [&](int kc) {
#pragma unroll
      for (int u = 0; u < XH_KC; ++u) {
        int kk = kc + u, jj = min(j0 + t, hcols - 1);
        int kr = min(kk, kin - 1);
        float v = H[(size_t)kr * ldh + jj];
        hr[u] = kk < kin ? v : 0.f;
      }
    };
    if (nch > 0) load_h(0);
    for (int c = 0; c < nch; ++c) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < XH_KC; ++u) Hs[u * XH_HS + t] = hr[u];
      __syncthreads();
      if (c + 1 < nch) load_h((c + 1) * XH_KC);
      const int kc = c * XH_KC;
      const int kl = min(XH_KC, kin - kc);
      // A: lane holds X(row l%16, k l/16); B: lane holds H(k l/16, col l%16)
      for (int kk = 0; kk < kl; kk += 4) {
        float av[RB];
#pragma unroll
        for (int a = 0; a < RB; ++a) av[a] = Xs[(a * 16 + (lane & 15)) * ldx + kc + kk + (lane >> 4)];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float bv = Hs[(kk + (lane >> 4)) * XH_HS + (wave * 4 + b) * 16 + (lane & 15)];
#pragma unroll
          for (int a = 0; a < RB; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv, acc[a][b], 0, 0, 0);
        }
      }
    }
    // result lane l, element e: row 4(l/16) + e, column l%16 of the block
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = j0 + (wave * 4 + b) * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = a * 16 + 4 * (lane >> 4) + e;
          if (r < nr && j < kout) {
            over |= iskv_st(Y + (size_t)(yo + i0 + r) * ldy + j, acc[a][b][e]);
            if (Ybf) Ybf[(size_t)(yo + i0 + r) * ldbf + j] = f2bf(acc[a][b][e]);
          }
        }
      }
  }
  iskv_latch_overflow<TY>(st, over);
}

// Same product with H held in registers (kin <= 288, kout <= 256): a
// 1024-thread workgroup, wave w owns output columns 16w .. 16w+15 and keeps
// its H slice as the B operand of v_mfma_f32_16x16x4f32 (lane l holds
// H(4kk + l/16, 16w + l%16) for kk < 72). Workgroups loop over 16-row blocks
// (block, block + grid, ...); each block's X rows are staged in LDS (double
// buffered, the next block's loads in flight during the current product)
// before any of its outputs is written, so in-place use stays safe.
constexpr int XR_LDX = 292; // LDS row stride (floats) of a staged X block

// One product's arguments (the paired launch takes two).
template <typename TX, typename TY>
struct XhJob {
  const TX* X1; int ld1; const float* X2; int ld2;
  Dim k1_d, kin_d; const float* H; int ldh, hcols; Dim kout_d, rows_d;
  TY* Y; int ldy; uint16_t* Ybf; int ldbf; int32_t* pos; const int32_t* pos_src; Dim yoff_d;
  const float4* Hf;
  int grid;  // workgroups of this product
};

// bx, gx: this workgroup's index among the product's gx workgroups.
template <int XR_KS, typename TX, typename TY>  // k steps of 4 held per lane: kin <= 4 XR_KS
__device__ __forceinline__ void xh_reg_body(const XhJob<TX, TY>& J, int bx, int gx, int32_t* st,
                                            float (*Xs)[16 * XR_LDX], const int64_t* __restrict__ bd) {
  const TX* X1 = J.X1; const int ld1 = J.ld1; const float* X2 = J.X2; const int ld2 = J.ld2;
  Dim k1_d = J.k1_d, kin_d = J.kin_d; const float* H = J.H; const int ldh = J.ldh, hcols = J.hcols;
  Dim kout_d = J.kout_d, rows_d = J.rows_d; TY* Y = J.Y; const int ldy = J.ldy; uint16_t* Ybf = J.Ybf;
  const int ldbf = J.ldbf; int32_t* pos = J.pos; const int32_t* pos_src = J.pos_src; Dim yoff_d = J.yoff_d;
  const float4* Hf = J.Hf;
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X1 = iskv_rb(X1, bdel);
  X2 = iskv_rb(X2, bdel);
  iskv_rb_dim(k1_d, bdel);
  iskv_rb_dim(kin_d, bdel);
  H = iskv_rb(H, bdel);
  Hf = iskv_rb(Hf, bdel);
  iskv_rb_dim(kout_d, bdel);
  iskv_rb_dim(rows_d, bdel);
  Y = iskv_rb(Y, bdel);
  Ybf = iskv_rb(Ybf, bdel);
  pos = iskv_rb(pos, bdel);
  pos_src = iskv_rb(pos_src, bdel);
  st = iskv_rb(st, bdel);
  iskv_rb_dim(yoff_d, bdel);
  constexpr int KW = 4 * XR_KS;                // staged columns (zero beyond kin)
  constexpr int PER = (16 * KW + 1023) / 1024;  // staged elements per thread
  const int k1 = dval(k1_d), kin = dval(kin_d), kout = dval(kout_d), rows = dval(rows_d);
  const int yo = dval(yoff_d);
  const int nblk = (rows + 15) / 16;
  if (bx >= nblk || kout <= 0 || kin <= 0) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = wave * 16 + (lane & 15);
  bool over = false;  // a saturated half store (fp16 coordinates only)
  float hreg[XR_KS];
  if (Hf) {  // H in operand order (eig_gather_kernel): 16-byte pieces
    static_assert(XR_KS % 4 == 0 && XR_KS / 4 <= XF_KQ, "operand-order H holds 72 k steps");
#pragma unroll
    for (int q = 0; q < XR_KS / 4; ++q) {
      const float4 f = Hf[(wave * XF_KQ + q) * 64 + lane];
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) hreg[4 * q + j] = 4 * (4 * q + j) + (lane >> 4) < kin ? fv[j] : 0.f;
    }
  } else {
    const int cc = min(col, hcols - 1);
    const char* hb = (const char*)H;
#pragma unroll
    for (int kk = 0; kk < XR_KS; ++kk) {
      const int kr = 4 * kk + (lane >> 4);
      const float v = *(const float*)(hb + 4u * (unsigned)(min(kr, kin - 1) * ldh + cc));
      hreg[kk] = kr < kin ? v : 0.f;
    }
  }
  // staged element u of this thread: e = t + 1024 u, row e / KW, column e % KW;
  // every load is issued from a valid address and masked when stored
  float xr[PER];
  auto load_x = [&](int blk) {
    const int i0 = blk * 16;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = min(t + 1024 * u, 16 * KW - 1), r = e / KW, c = e % KW;
      const int row = min(i0 + r, rows - 1);
      if constexpr (std::is_same<TX, float>::value) {
        const float* src = c < k1 ? X1 + (size_t)row * ld1 + c
                                  : (c < kin ? X2 + (size_t)row * ld2 + (c - k1) : X1 + (size_t)row * ld1);
        xr[u] = *src;
      } else {  // 2-byte rows are only ever the whole input (k1 = kin)
        xr[u] = iskv_ld(X1 + (size_t)row * ld1 + min(c, k1 - 1));
      }
    }
  };
  load_x(bx);
  int buf = 0;
  for (int blk = bx; blk < nblk; blk += gx) {
    float* xs = Xs[buf];
    const int i0 = blk * 16;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + 1024 * u, r = e / KW, c = e % KW;
      if (e < 16 * KW) xs[r * XR_LDX + c] = (c < kin && i0 + r < rows) ? xr[u] : 0.f;
    }
    __syncthreads();
    if (blk + gx < nblk) load_x(blk + gx);
    v4f_t acc = {0.f, 0.f, 0.f, 0.f};
    const float* xa = xs + (lane & 15) * XR_LDX + (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < XR_KS; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * kk], hreg[kk], acc, 0, 0, 0);
    if (col < kout) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + 4 * (lane >> 4) + e;
        if (row < rows) {
          over |= iskv_st(Y + (size_t)(yo + row) * ldy + col, acc[e]);
          if (Ybf) Ybf[(size_t)(yo + row) * ldbf + col] = f2bf(acc[e]);
        }
      }
    }
    if (pos && t < 16 && i0 + t < rows) pos[yo + i0 + t] = pos_src[i0 + t];
    buf ^= 1;
  }
  iskv_latch_overflow<TY>(st, over);
}

template <int XR_KS, typename TX, typename TY>
__global__ __launch_bounds__(1024) void xh_reg_kernel(XhJob<TX, TY> J, int32_t* st, const int64_t* __restrict__ bd) {
  __shared__ float Xs[2][16 * XR_LDX];
  xh_reg_body<XR_KS>(J, blockIdx.x, gridDim.x, st, Xs, bd);
}

// Two independent products in one launch: workgroups [0, A.grid) run A, the
// rest run B (the merge's new rows and basis update, which share H).
template <int XR_KS, typename TX, typename TY>
__global__ __launch_bounds__(1024) void xh_reg2_kernel(XhJob<TX, TY> A, XhJob<TX, TY> B, int32_t* st,
                                                       const int64_t* __restrict__ bd) {
  __shared__ float Xs[2][16 * XR_LDX];
  if ((int)blockIdx.x < A.grid) xh_reg_body<XR_KS>(A, blockIdx.x, A.grid, st, Xs, bd);
  else xh_reg_body<XR_KS>(B, blockIdx.x - A.grid, B.grid, st, Xs, bd);
}

// The coordinate update C <- C H over all n rows (C n x kin, in place; H
// kin x kout, kin, kout <= 256) on the bf16 matrix cores with split operands:
// x = x_h + x_l and h = h_h + h_l, each part a bf16 (x_h = bf16(x),
// x_l = bf16(x - x_h)), and
//   x . h ~ x_h . h_h + x_h . h_l + x_l . h_h
// in fp32 accumulation (v_mfma_f32_16x16x32_bf16). The dropped x_l . h_l and
// the parts' own rounding leave about 2^-16 of |x| |h| per product, against
// 2^-24 for fp32 products; three bf16 products cost a fifth of the fp32
// matrix-core time at r = 256, which puts the update under its HBM time.
// A 1024-thread workgroup: wave w owns output columns 16 w .. 16 w + 15 and
// keeps their split H as the B operands (lane l: column l % 16, k 32 s +
// 8 (l / 16) .. +7, for s < 8), read as prepared by split_h_kernel (once per
// merge, in operand order: every lane loads 16 contiguous 16-byte pieces
// instead of gathering 64 strided values). Rows go in 16-row
// blocks (block, block + grid, ...), loaded a chunk of blocks at a time,
// each split into two bf16 images in LDS (two staging buffers alternate, one
// barrier per block) and multiplied; a block's rows are all read before any
// of its outputs is written, so the update is in place.
// 2-byte stored coordinates (TX = uint16_t) are exact in bf16: x_l = 0 and
// the x_l . h_h product is skipped.
constexpr int XB_LD = 256 + 8;  // LDS row stride (bf16) of a staged block image
constexpr int XB_CH = 8;        // blocks whose rows are loaded together

// Split fragments of H for xh_bf3_kernel: fragment (w, s) of lane l holds
// the 8 bf16 of column 16 w + l % 16, rows 32 s + 8 (l / 16) .. +7 (zero past
// kin and kout), hi parts at Hs[(w NS + s) 64 + l], lo parts NW NS 64 uint4
// further (NW = r_max / 16 column blocks, NS = r_max / 32 depth steps).
__global__ __launch_bounds__(256) void split_h_kernel(const float* __restrict__ H, int ldh, Dim kin_d, Dim kout_d,
                                                      int NW, int NS, uint4* Hs, const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  H = iskv_rb(H, bdel);
  Hs = iskv_rb(Hs, bdel);
  iskv_rb_dim(kin_d, bdel);
  iskv_rb_dim(kout_d, bdel);
  const int kin = dval(kin_d), kout = dval(kout_d);
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g >= NW * NS * 64) return;
  const int lane = g & 63, sk = (g >> 6) % NS, w = (g >> 6) / NS;
  const int col = 16 * w + (lane & 15);
  float hv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 32 * sk + 8 * (lane >> 4) + j;
    hv[j] = (k < kin && col < kout) ? H[(size_t)k * ldh + col] : 0.f;
  }
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ph[j] = pk_bf16(hv[2 * j], hv[2 * j + 1]);
    const float h0 = __uint_as_float(ph[j] << 16), h1 = __uint_as_float(ph[j] & 0xffff0000u);
    pl[j] = pk_bf16(hv[2 * j] - h0, hv[2 * j + 1] - h1);
  }
  Hs[g] = uint4{ph[0], ph[1], ph[2], ph[3]};
  Hs[NW * NS * 64 + g] = uint4{pl[0], pl[1], pl[2], pl[3]};
}

template <typename TX>
__global__ __launch_bounds__(1024) void xh_bf3_kernel(TX* X, int ldx, Dim kin_d, const uint4* __restrict__ Hs, int NW,
                                                      int NS, Dim kout_d, Dim rows_d, int32_t* st,
                                                      const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X = iskv_rb(X, bdel);
  st = iskv_rb(st, bdel);
  Hs = iskv_rb(Hs, bdel);
  iskv_rb_dim(kin_d, bdel);
  iskv_rb_dim(kout_d, bdel);
  iskv_rb_dim(rows_d, bdel);
  // fp32 and fp16 rows need the low bf16 part (fp16 carries 11 significant
  // bits); bf16 rows are exact in the high part
  constexpr bool SPLIT_X = !std::is_same<TX, uint16_t>::value;
  bool over = false;  // a saturated half store (fp16 coordinates only)
  const int kin = dval(kin_d), kout = dval(kout_d), rows = dval(rows_d);
  const int nblk = (rows + 15) / 16;
  if ((int)blockIdx.x >= nblk || kout <= 0 || kin <= 0) return;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][2][16 * XB_LD];  // [buffer][hi, lo]
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = wave * 16 + (lane & 15);
  // split H operands: hh[s], hl[s] = 8 bf16 of column col, k 32 s + 8 (l / 16) ..
  // (depth steps past NS and waves past NW are zero; those waves only stage rows)
  v8bf hh[8], hl[8];
#pragma unroll
  for (int sk = 0; sk < 8; ++sk) {
    const bool in = sk < NS && wave < NW;
    const uint4 a = in ? Hs[(wave * NS + sk) * 64 + lane] : uint4{0u, 0u, 0u, 0u};
    const uint4 b = in ? Hs[(NW * NS + wave * NS + sk) * 64 + lane] : uint4{0u, 0u, 0u, 0u};
    hh[sk] = __builtin_bit_cast(v8bf, a);
    hl[sk] = __builtin_bit_cast(v8bf, b);
  }
  // block staging: thread t holds row t / 64, columns 4 (t % 64) .. +3 of
  // each 16-row block (rows past `rows` and columns past kin read as zero).
  // A workgroup's blocks go in chunks of XB_CH: the rows of the whole chunk
  // are loaded first, so the memory latency is paid once per chunk.
  const int sr = t >> 6, sc = (t & 63) * 4;
  float4 xr[XB_CH];
  auto load_x = [&](int u, int blk) {
    const int row = min(blk * 16 + sr, rows - 1);
    if constexpr (std::is_same<TX, float>::value) {
      xr[u] = *(const float4*)(X + (size_t)row * ldx + sc);
    } else if constexpr (std::is_same<TX, _Float16>::value) {
      typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
      const h4_t v = *(const h4_t*)(X + (size_t)row * ldx + sc);
      xr[u] = float4{(float)v.x, (float)v.y, (float)v.z, (float)v.w};
    } else {
      const uint2 v = *(const uint2*)(X + (size_t)row * ldx + sc);
      xr[u] = float4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u)};
    }
  };
  int buf = 0;
  for (int c0 = blockIdx.x; c0 < nblk; c0 += XB_CH * gridDim.x) {
#pragma unroll
  for (int u = 0; u < XB_CH; ++u)
    if (c0 + u * (int)gridDim.x < nblk) load_x(u, c0 + u * gridDim.x);
#pragma unroll
  for (int u = 0; u < XB_CH; ++u) {
    const int blk = c0 + u * gridDim.x;
    if (blk >= nblk) break;
    const int i0 = blk * 16;
    {
      const bool rv = i0 + sr < rows;
      const float4 xv = xr[u];
      const float x0 = (rv && sc < kin) ? xv.x : 0.f, x1 = (rv && sc + 1 < kin) ? xv.y : 0.f;
      const float x2 = (rv && sc + 2 < kin) ? xv.z : 0.f, x3 = (rv && sc + 3 < kin) ? xv.w : 0.f;
      const uint32_t h01 = pk_bf16(x0, x1), h23 = pk_bf16(x2, x3);
      *(uint2*)(&Xs[buf][0][sr * XB_LD + sc]) = uint2{h01, h23};
      if constexpr (SPLIT_X) {
        const uint32_t l01 = pk_bf16(x0 - __uint_as_float(h01 << 16), x1 - __uint_as_float(h01 & 0xffff0000u));
        const uint32_t l23 = pk_bf16(x2 - __uint_as_float(h23 << 16), x3 - __uint_as_float(h23 & 0xffff0000u));
        *(uint2*)(&Xs[buf][1][sr * XB_LD + sc]) = uint2{l01, l23};
      }
    }
    __syncthreads();
    v4f_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xh = &Xs[buf][0][(lane & 15) * XB_LD + 8 * (lane >> 4)];
    const uint16_t* xl = &Xs[buf][1][(lane & 15) * XB_LD + 8 * (lane >> 4)];
#pragma unroll
    for (int sk = 0; sk < 8; ++sk) {
      const v8bf ah = __builtin_bit_cast(v8bf, *(const uint4*)(xh + 32 * sk));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, hh[sk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, hl[sk], acc, 0, 0, 0);
      if constexpr (SPLIT_X) {
        const v8bf al = __builtin_bit_cast(v8bf, *(const uint4*)(xl + 32 * sk));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, hh[sk], acc, 0, 0, 0);
      }
    }
    // result lane l, element e: row 4 (l / 16) + e, column l % 16 of the wave's block
    if (col < kout) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = i0 + 4 * (lane >> 4) + e;
        if (row < rows) over |= iskv_st(X + (size_t)row * ldx + col, acc[e]);
      }
    }
    buf ^= 1;
  }
  }
  iskv_latch_overflow<TX>(st, over);
}

// Streaming form of the same update for r_max = 256 (ldx = 256): a
// 512-thread workgroup per CU, wave w owning output columns 32 w .. 32 w + 31
// (two 16-column blocks of split H as A operands, so each lane's result is
// four consecutive columns of one row: one 16- or 8-byte store per block and
// column block). The workgroup's 16-row blocks b0, b0 + G, ... pass through a
// three-stage pipeline: the rows of block j + 2 are requested while block
// j + 1 is split into the idle LDS image and block j is multiplied, with one
// barrier per block. Every block issues the same memory operations (loads of
// a block past the workgroup's last re-read that block and are discarded;
// stores of rows past the end are dropped by the descriptor, and a block
// always has at least one row in range), and the prologue issues, after the
// rows of the first two blocks, the stores of one block into a scratch line
// that nothing reads, so the wait counts at the head of the loop equal the
// steady state's: the in-order counter waits for exactly the block in use.
// Columns in [kout, r_max) receive zeros (H is zero there).
constexpr int XS_NT = 512;  // threads of the streaming update

template <typename TX>
__global__ __launch_bounds__(XS_NT) void xh_bf3s_kernel(TX* X, int ldx, Dim kin_d, const uint4* __restrict__ Hs,
                                                        int NW, int NS, Dim kout_d, Dim rows_d, int32_t* st,
                                                        float* scratch, int scratch_lines,
                                                        const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X = iskv_rb(X, bdel);
  st = iskv_rb(st, bdel);
  Hs = iskv_rb(Hs, bdel);
  scratch = iskv_rb(scratch, bdel);
  iskv_rb_dim(kin_d, bdel);
  iskv_rb_dim(kout_d, bdel);
  iskv_rb_dim(rows_d, bdel);
  constexpr bool SPLIT_X = !std::is_same<TX, uint16_t>::value;
  constexpr int ES = (int)sizeof(TX);
  const int kin = dval(kin_d), kout = dval(kout_d), rows = dval(rows_d);
  const int nblk = (rows + 15) / 16;
  const int G = gridDim.x, b0 = blockIdx.x;
  if (b0 >= nblk || kout <= 0 || kin <= 0) return;
  const int nb = (nblk - b0 + G - 1) / G;  // blocks b0 + j G, j < nb
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][SPLIT_X ? 2 : 1][16 * XB_LD];  // [buffer][hi, lo]
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  bool over = false;  // a saturated half store (fp16 coordinates only)
  // staging: thread t holds row t / 32, columns 8 (t % 32) .. +7 of a block
  const int sr = t >> 5, sc = (t & 31) * 8;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)((size_t)rows * ldx * ES), 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)scratch, (short)0,
                                                                      scratch_lines * 128, 0x00020000);
  const uint32_t soff = (uint32_t)((b0 % scratch_lines) * 128);
  // rows in flight: fp32 rows as two float4, 2-byte rows as one uint4 of raw bits
  uint4 ring[2][ES == 4 ? 2 : 1];
  auto load = [&](auto slot_c, int j) {
    constexpr int slot = decltype(slot_c)::value;
    const int row = min((b0 + min(j, nb - 1) * G) * 16 + sr, rows - 1);
    const uint32_t o = (uint32_t)(((size_t)row * ldx + sc) * ES);
    ring[slot][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
    if constexpr (ES == 4)
      ring[slot][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, o + 16, 0, 0));
  };
  // split H operands of column blocks 2 w and 2 w + 1 (past NW: zero)
  const __amdgpu_buffer_rsrc_t rh =
      __builtin_amdgcn_make_buffer_rsrc((void*)Hs, (short)0, NW * NS * 64 * 16 * 2, 0x00020000);
  v8bf hh[2][8], hl[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int sk = 0; sk < 8; ++sk) {
      const int w = 2 * wave + q;
      const bool in = sk < NS && w < NW;
      const uint32_t oa = in ? (uint32_t)(((w * NS + sk) * 64 + lane) * 16) : 0x80000000u;
      const uint32_t ob = in ? (uint32_t)(((NW * NS + w * NS + sk) * 64 + lane) * 16) : 0x80000000u;
      hh[q][sk] = __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(rh, oa, 0, 0));
      hl[q][sk] = __builtin_bit_cast(v8bf, __builtin_amdgcn_raw_buffer_load_b128(rh, ob, 0, 0));
    }
  __builtin_amdgcn_sched_barrier(0);  // H is requested first, so it has arrived once block 0 has
  load(std::integral_constant<int, 0>{}, 0);
  load(std::integral_constant<int, 1>{}, 1);
  __builtin_amdgcn_raw_buffer_store_b128(v4u{0u, 0u, 0u, 0u}, rs, soff, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(v4u{0u, 0u, 0u, 0u}, rs, soff + 64, 0, 0);
  // split the rows of a slot into the LDS images (rows past the end and
  // columns >= kin as zero)
  auto stage = [&](auto slot_c, int j, int buf) {
    constexpr int slot = decltype(slot_c)::value;
    const bool rv = (b0 + j * G) * 16 + sr < rows;
    float x[8];
    if constexpr (ES == 4) {
      const uint4 a = ring[slot][0], b = ring[slot][1];
      const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(u[e]);
    } else if constexpr (std::is_same<TX, _Float16>::value) {
      const uint4 a = ring[slot][0];
      const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const h2_t hv = __builtin_bit_cast(h2_t, u[e]);
        x[2 * e] = (float)hv.x;
        x[2 * e + 1] = (float)hv.y;
      }
    } else {
      const uint4 a = ring[slot][0];
      const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = __uint_as_float(u[e] << 16);
        x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = (rv && sc + 2 * e < kin) ? x[2 * e] : 0.f;
      const float b = (rv && sc + 2 * e + 1 < kin) ? x[2 * e + 1] : 0.f;
      hi[e] = pk_bf16(a, b);
      lo[e] = pk_bf16(a - __uint_as_float(hi[e] << 16), b - __uint_as_float(hi[e] & 0xffff0000u));
    }
    *(uint4*)(&Xs[buf][0][sr * XB_LD + sc]) = uint4{hi[0], hi[1], hi[2], hi[3]};
    if constexpr (SPLIT_X) *(uint4*)(&Xs[buf][SPLIT_X ? 1 : 0][sr * XB_LD + sc]) = uint4{lo[0], lo[1], lo[2], lo[3]};
  };
  stage(std::integral_constant<int, 0>{}, 0, 0);
  __syncthreads();
  const int cw = 32 * wave + 4 * (lane >> 4);  // this lane's first output column (column block 0)

  auto process = [&](auto slot_c, int j) {
    constexpr int slot = decltype(slot_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    const int buf = j & 1;
    v8bf ah[8], al[8];
    const uint16_t* xh = &Xs[buf][0][(lane & 15) * XB_LD + 8 * (lane >> 4)];
#pragma unroll
    for (int sk = 0; sk < 8; ++sk) {
      ah[sk] = __builtin_bit_cast(v8bf, *(const uint4*)(xh + 32 * sk));
      if constexpr (SPLIT_X) {
        const uint16_t* xl = &Xs[buf][SPLIT_X ? 1 : 0][(lane & 15) * XB_LD + 8 * (lane >> 4)];
        al[sk] = __builtin_bit_cast(v8bf, *(const uint4*)(xl + 32 * sk));
      }
    }
    stage(std::integral_constant<int, slot ^ 1>{}, j + 1, buf ^ 1);
    load(slot_c, j + 2);
    v4f_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int sk = 0; sk < 8; ++sk) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hh[q][sk], ah[sk], acc[q], 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hl[q][sk], ah[sk], acc[q], 0, 0, 0);
        if constexpr (SPLIT_X) acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hh[q][sk], al[sk], acc[q], 0, 0, 0);
      }
    }
    // result lane l, element e: row i0 + l % 16, column cw + 16 q + e
    const int row = (b0 + j * G) * 16 + (lane & 15);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t o = row < rows ? (uint32_t)(((size_t)row * ldx + cw + 16 * q) * ES) : 0x80000000u;
      if constexpr (ES == 4) {
        const v4u v = __builtin_bit_cast(v4u, acc[q]);
        __builtin_amdgcn_raw_buffer_store_b128(v, rx, o, 0, 0);
      } else {
        uint32_t p0, p1;
        if constexpr (std::is_same<TX, _Float16>::value) {
#pragma unroll
          for (int e = 0; e < 4; ++e) over |= row < rows && iskv_f16_over(acc[q][e]);
          p0 = __builtin_bit_cast(uint32_t, h2_t{iskv_to_f16(acc[q][0]), iskv_to_f16(acc[q][1])});
          p1 = __builtin_bit_cast(uint32_t, h2_t{iskv_to_f16(acc[q][2]), iskv_to_f16(acc[q][3])});
        } else {
          p0 = pk_bf16(acc[q][0], acc[q][1]);
          p1 = pk_bf16(acc[q][2], acc[q][3]);
        }
        __builtin_amdgcn_raw_buffer_store_b64(v2u{p0, p1}, rx, o, 0, 0);
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  int jb = 0;
  for (; jb + 2 <= nb; jb += 2) {
    process(std::integral_constant<int, 0>{}, jb);
    process(std::integral_constant<int, 1>{}, jb + 1);
  }
  if (jb < nb) process(std::integral_constant<int, 0>{}, jb);
  iskv_latch_overflow<TX>(st, over);
}

// Launch Y = [X1 | X2] H over `rows_host` rows (an upper bound when rows_d is
// a device value); kin_max bounds kin for the LDS layout.
template <typename TX, typename TY>
static void xh_launch(hipStream_t s, const int64_t* bd, int bc, int rows_host, const TX* X1, int ld1, const float* X2, int ld2,
                      Dim k1, Dim kin, int kin_max, const float* H, int ldh, int hcols, Dim kout,
                      Dim rows, TY* Y, int ldy, uint16_t* Ybf, int ldbf, int32_t* pos = nullptr,
                      const int32_t* pos_src = nullptr, bool prefer16 = false, Dim yoff = hdim(0),
                      int32_t* st = nullptr, const float4* Hf = nullptr) {
  const int ldx = xh_ldx(kin_max);
  if (kin_max <= 288 && hcols <= 256) {
    const int nblk = (rows_host + 15) / 16;
    const int grid = nblk < 256 ? nblk : 256;
    if (grid > 0) {
      const XhJob<TX, TY> J = {X1, ld1, X2, ld2, k1, kin, H, ldh, hcols, kout, rows, Y, ldy, Ybf, ldbf, pos, pos_src,
                               yoff, Hf, grid};
      if (kin_max <= 256)
        hipLaunchKernelGGL((xh_reg_kernel<64, TX, TY>), bz(dim3(grid), bc), dim3(1024), 0, s, J, st, bd);
      else
        hipLaunchKernelGGL((xh_reg_kernel<72, TX, TY>), bz(dim3(grid), bc), dim3(1024), 0, s, J, st, bd);
    }
    return;
  }
  if (!prefer16 && xh_lds_bytes(32, kin_max) <= 80 * 1024) {
    hipLaunchKernelGGL((xh_mfma_kernel<32, TX, TY>), bz(dim3((rows_host + 31) / 32), bc), dim3(256),
                       xh_lds_bytes(32, kin_max), s, X1, ld1, X2, ld2, k1, kin, H, ldh, hcols, kout,
                       rows, Y, ldy, Ybf, ldbf, ldx, pos, pos_src, yoff, st, bd);
  } else {
    hipLaunchKernelGGL((xh_mfma_kernel<16, TX, TY>), bz(dim3((rows_host + 15) / 16), bc), dim3(256),
                       xh_lds_bytes(16, kin_max), s, X1, ld1, X2, ld2, k1, kin, H, ldh, hcols, kout,
                       rows, Y, ldy, Ybf, ldbf, ldx, pos, pos_src, yoff, st, bd);
  }
}

// Commit a merge: sigma <- sigma+, k <- r', n += b, folded += b.
__global__ void merge_commit_kernel(float* sigma, const float* __restrict__ sig_new, int32_t* st,
                                    int b, int r_max,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  sigma = iskv_rb(sigma, bdel);
  sig_new = iskv_rb(sig_new, bdel);
  st = iskv_rb(st, bdel);
  const int kout = st[ST_KNEW];
  for (int j = threadIdx.x; j < r_max; j += blockDim.x) sigma[j] = j < kout ? sig_new[j] : 0.f;
  __syncthreads();
  if (threadIdx.x == 0) {
    st[ST_K] = kout;
    st[ST_N] += b;
    st[ST_FOLDED] += b;
  }
}

// Frozen-basis merge (iS-KV notes §6.4 / §8 baseline): append the new rows'
// coordinates Q = F B (b x k, columns past k zero) and positions at row n,
// then n += b. One workgroup per path: every thread reads n before thread 0
// advances it. Non-finite coordinates are latched like the full merge's input.
template <typename TC>
__global__ __launch_bounds__(256) void frozen_append_kernel(const float* __restrict__ Q, int ldq,
                                                            const int32_t* __restrict__ pos_F, int b, TC* C,
                                                            int ldc, int32_t* pos, int32_t* st,
                                                            const int64_t* __restrict__ bd) {
  const int64_t d = bd ? bd[blockIdx.z] : 0;
  Q = iskv_rb(Q, d);
  pos_F = iskv_rb(pos_F, d);
  C = iskv_rb(C, d);
  pos = iskv_rb(pos, d);
  st = iskv_rb(st, d);
  const int n = st[ST_N], k = st[ST_K];
  bool bad = false, over = false;
  for (int e = threadIdx.x; e < b * ldc; e += blockDim.x) {
    const int i = e / ldc, j = e % ldc;
    const float v = j < k ? Q[(size_t)i * ldq + j] : 0.f;
    bad |= !isfinite(v);
    over |= iskv_st(C + (size_t)(n + i) * ldc + j, v);
  }
  for (int i = threadIdx.x; i < b; i += blockDim.x) pos[n + i] = pos_F[i];
  if (bad) atomicOr(&st[ST_STATUS], ISKV_DEV_NONFINITE);
  iskv_latch_overflow<TC>(st, over);
  __syncthreads();
  if (threadIdx.x == 0) {
    st[ST_N] = n + b;
    st[ST_FOLDED] += b;
  }
}

// Copy k (or another slot) into ST_JM so the eigensolver knows its order.
__global__ void set_jm_kernel(int32_t* st, int from_slot,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  st = iskv_rb(st, bdel);
  st[ST_JM] = st[from_slot];
}

// ----------------------------------------------------------------------------
// Re-orthogonalisation helpers.
// Partial Gram of the columns of X (rows x k, fp32) over a row chunk, fp64:
// G_part[s][i][j] = sum_{rows in chunk s} X[r, i] X[r, j]. Grid: (tiles of
// 16x16 over k x k, chunks). 256 threads.
template <typename TX>
__global__ __launch_bounds__(256) void gram_partial_kernel(const TX* __restrict__ X, int ldx,
                                                           Dim rows_d, const int32_t* st,
                                                           double* Gpart, int ldg,
                                                           int rows_per_chunk,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X = iskv_rb(X, bdel);
  iskv_rb_dim(rows_d, bdel);
  st = iskv_rb(st, bdel);
  Gpart = iskv_rb(Gpart, bdel);
  const int k = st[ST_K];
  const int rows = dval(rows_d);
  const int tiles = (k + 15) / 16;
  const int ti = blockIdx.x / tiles, tj = blockIdx.x % tiles;
  if (ti >= tiles) return;
  const int i = ti * 16 + (threadIdx.x >> 4), j = tj * 16 + (threadIdx.x & 15);
  const int r0 = blockIdx.y * rows_per_chunk, r1 = min(rows, r0 + rows_per_chunk);
  __shared__ float Xi[64][17], Xj[64][17];
  double acc = 0.0;
  for (int rb = r0; rb < r1; rb += 64) {
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
      int rr = idx >> 4, cc = idx & 15;
      int row = rb + rr;
      int ci = ti * 16 + cc, cj = tj * 16 + cc;
      Xi[rr][cc] = (row < r1 && ci < k) ? iskv_ld(X + (size_t)row * ldx + ci) : 0.f;
      Xj[rr][cc] = (row < r1 && cj < k) ? iskv_ld(X + (size_t)row * ldx + cj) : 0.f;
    }
    __syncthreads();
    for (int rr = 0; rr < 64; ++rr)
      acc = fma((double)Xi[rr][threadIdx.x >> 4], (double)Xj[rr][threadIdx.x & 15], acc);
    __syncthreads();
  }
  if (i < k && j < k) Gpart[((size_t)blockIdx.y * ldg + i) * ldg + j] = acc;
}

// Sum the partial Grams: G_C = sum of the C slices, G_B = the B slice, both
// into m_max-ld fp64 matrices, and Z0 = 1.5 I - 0.5 G_B (first Newton-Schulz
// step towards G_B^(-1/2)). Grid-stride over k x k.
__global__ __launch_bounds__(256) void reorth_sum_kernel(const double* __restrict__ Gpart, int nchunks,
                                                         int ldg, double* GC, double* GB, double* Z0,
                                                         int ld, const int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  Gpart = iskv_rb(Gpart, bdel);
  GC = iskv_rb(GC, bdel);
  GB = iskv_rb(GB, bdel);
  Z0 = iskv_rb(Z0, bdel);
  st = iskv_rb(st, bdel);
  const int k = st[ST_K];
  const size_t tot = (size_t)k * k;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / k), j = (int)(e % k);
    double a = 0.0;
    for (int c = 0; c < nchunks; ++c) a += Gpart[((size_t)c * ldg + i) * ldg + j];
    double gb = Gpart[((size_t)nchunks * ldg + i) * ldg + j];
    GC[(size_t)i * ld + j] = a;
    GB[(size_t)i * ld + j] = gb;
    Z0[(size_t)i * ld + j] = (i == j ? 1.5 : 0.0) - 0.5 * gb;
  }
}

// Y[:, t] = V[:, order[t]] (fp64, sorted eigenvectors). Grid-stride.
__global__ __launch_bounds__(256) void permute_cols_kernel(const double* __restrict__ V,
                                                           const int32_t* __restrict__ order,
                                                           double* Y, int ld, const int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  V = iskv_rb(V, bdel);
  order = iskv_rb(order, bdel);
  Y = iskv_rb(Y, bdel);
  st = iskv_rb(st, bdel);
  const int k = st[ST_JM];
  const size_t tot = (size_t)k * k;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / k), t = (int)(e % k);
    Y[(size_t)i * ld + t] = V[(size_t)i * ld + min(max(order[t], 0), k - 1)];
  }
}

// fp64 (ld) -> fp32 (ld r_max) for the two k x k transforms.
__global__ __launch_bounds__(256) void to_f32_kernel(const double* __restrict__ X1,
                                                     const double* __restrict__ X2, int ld, float* Y1,
                                                     float* Y2, int ldy, const int32_t* st,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X1 = iskv_rb(X1, bdel);
  X2 = iskv_rb(X2, bdel);
  Y1 = iskv_rb(Y1, bdel);
  Y2 = iskv_rb(Y2, bdel);
  st = iskv_rb(st, bdel);
  const int k = st[ST_K];
  const size_t tot = (size_t)k * k;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / k), j = (int)(e % k);
    Y1[(size_t)i * ldy + j] = (float)X1[(size_t)i * ld + j];
    Y2[(size_t)i * ldy + j] = (float)X2[(size_t)i * ld + j];
  }
}

__global__ void reorth_commit_kernel(float* sigma, const float* __restrict__ sig_new, int32_t* st,
                                     int r_max,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  sigma = iskv_rb(sigma, bdel);
  sig_new = iskv_rb(sig_new, bdel);
  st = iskv_rb(st, bdel);
  const int k = st[ST_K];
  for (int j = threadIdx.x; j < r_max; j += blockDim.x) sigma[j] = j < k ? sig_new[j] : 0.f;
}

}  // namespace

// Copy a caller matrix (ld m) into the workspace (ld m_max) and set ST_JM.
__global__ __launch_bounds__(256) void load_sym_kernel(const double* __restrict__ Ain, int m, double* A,
                                                       int ld, int32_t* st) {
  const size_t tot = (size_t)m * m;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / m), j = (int)(e % m);
    A[(size_t)i * ld + j] = Ain[e];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) st[ST_JM] = m;
}

// lam[t] = S[order[t], order[t]], Vout[:, t] = V[:, order[t]] (ld m).
__global__ __launch_bounds__(256) void store_sym_kernel(const double* __restrict__ S,
                                                        const double* __restrict__ V, int ld,
                                                        const int32_t* __restrict__ order, int m,
                                                        double* lam, double* Vout) {
  const size_t tot = (size_t)m * m;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < tot; e += (size_t)gridDim.x * 256) {
    int i = (int)(e / m), t = (int)(e % m);
    int o = min(max(order[t], 0), m - 1);
    Vout[e] = V[(size_t)i * ld + o];
    if (i == 0) lam[t] = S[(size_t)o * ld + o];
  }
}

// ============================================================================
// Host launchers.

// out (M x N) = alpha * X (M x K) op(Y) + beta * Z, split over K.
// Skinny products on fp32 MFMA (v_mfma_f32_16x16x4f32), one launch each:
//   out[i, j] = alpha * sum_k X[i, k] Y'(k, j) + beta * Z[i, j],  i < M (<= 64),
//   Y'(k, j) = TY ? Y[j, k] : Y[k, j].
// A workgroup of NW waves owns one 16 x 16 output block; wave w takes the
// depth chunks of 16 at w, w + NW, ... and issues the loads of up to SK_CPW
// chunks before their MFMAs, so a wave waits for memory about once per
// NW * SK_CPW chunks (the whole depth at the merge shapes); the partial
// blocks are summed through LDS. Inside a chunk, lane l (row or column l%16,
// group g = l/16) takes depths 16 s + 4 g + q for MFMA step q: the summation
// order over k is permuted so that each lane's four operands are consecutive
// in memory. Depths >= K, rows >= M and columns >= N are masked or dropped.
// VEC (X rows, and Y rows when TY, 16-byte aligned with a leading dimension
// divisible by 4): a lane's four consecutive depths come in one 16-byte load.
constexpr int SK_CPW = 4;
template <bool TY, int NW, bool VEC>
__global__ __launch_bounds__(64 * NW) void skinny_mfma_kernel(const float* __restrict__ X, int ldx,
                                                               const float* __restrict__ Y, int ldy, int M,
                                                               int Nmax, Dim Nd, Dim Kd, float alpha,
                                                               float beta, const float* Z, int ldz,
                                                               float* out, int ldo,
    const int64_t* __restrict__ bd) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  X = iskv_rb(X, bdel);
  Y = iskv_rb(Y, bdel);
  iskv_rb_dim(Nd, bdel);
  iskv_rb_dim(Kd, bdel);
  Z = iskv_rb(Z, bdel);
  out = iskv_rb(out, bdel);
  const int N = dval(Nd), K = dval(Kd);
  const int j0 = blockIdx.x * 16, i0 = blockIdx.y * 16;
  if (j0 >= N) return;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int row = min(i0 + r, M - 1), col = min(j0 + r, Nmax - 1);
  const float* xr = X + (size_t)row * ldx;
  v4f_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nch = (K + 15) / 16;
  for (int c0 = wave; c0 < nch; c0 += NW * SK_CPW) {
    float av[SK_CPW][4], bv[SK_CPW][4];
#pragma unroll
    for (int u = 0; u < SK_CPW; ++u) {
      const int kb = (c0 + NW * u) * 16 + 4 * g;
      if (VEC && kb + 4 <= K) {
        const float4 a = *(const float4*)(xr + kb);
        av[u][0] = a.x; av[u][1] = a.y; av[u][2] = a.z; av[u][3] = a.w;
        if constexpr (TY) {
          const float4 y = *(const float4*)(Y + (size_t)col * ldy + kb);
          bv[u][0] = y.x; bv[u][1] = y.y; bv[u][2] = y.z; bv[u][3] = y.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) bv[u][q] = Y[(size_t)(kb + q) * ldy + col];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = kb + q, kc = min(k, K - 1);
          const float a = xr[kc];
          const float bb = TY ? Y[(size_t)col * ldy + kc] : Y[(size_t)kc * ldy + col];
          av[u][q] = k < K ? a : 0.f;
          bv[u][q] = k < K ? bb : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < SK_CPW; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][q], bv[u][q], acc, 0, 0, 0);
  }
  __shared__ float red[NW - 1][4][64];
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave > 0) return;
  // result lane l, element e: row 4(l/16) + e, column l%16
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = acc[e];
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) v += red[w][e][lane];
    const int i = i0 + 4 * g + e, j = j0 + r;
    if (i < M && j < N) {
      float o = alpha * v;
      if (beta != 0.f) o += beta * Z[(size_t)i * ldz + j];
      out[(size_t)i * ldo + j] = o;
    }
  }
}

// Waves per workgroup: enough that the whole depth (Kmax) is in flight at once.
template <bool TY>
static void skinny(isvd_handle* h, int M, int Nmax, const float* X, int ldx, const float* Y, int ldy,
                   Dim N, int Kmax, float alpha, float beta, const float* Z, int ldz, float* out,
                   int ldo) {
  Dim K = TY ? ddim(h->w.st + ST_K) : hdim(Kmax);
  dim3 grid((Nmax + 15) / 16, (M + 15) / 16);
  const int nch = (Kmax + 15) / 16;
  // one path: its pointers are checked here (batched paths are rebased on the
  // device by offsets the host does not inspect, so they keep scalar loads)
  const bool vec = h->bcount == 1 && ldx % 4 == 0 && ((uintptr_t)X & 15) == 0 &&
                   (!TY || (ldy % 4 == 0 && ((uintptr_t)Y & 15) == 0));
  if (nch > 4 * SK_CPW) {
    if (vec)
      hipLaunchKernelGGL((skinny_mfma_kernel<TY, 16, true>), bz(grid, h->bcount), dim3(1024), 0, h->stream, X, ldx,
                         Y, ldy, M, Nmax, N, K, alpha, beta, Z, ldz, out, ldo, h->bd);
    else
      hipLaunchKernelGGL((skinny_mfma_kernel<TY, 16, false>), bz(grid, h->bcount), dim3(1024), 0, h->stream, X, ldx,
                         Y, ldy, M, Nmax, N, K, alpha, beta, Z, ldz, out, ldo, h->bd);
  } else {
    if (vec)
      hipLaunchKernelGGL((skinny_mfma_kernel<TY, 4, true>), bz(grid, h->bcount), dim3(256), 0, h->stream, X, ldx, Y,
                         ldy, M, Nmax, N, K, alpha, beta, Z, ldz, out, ldo, h->bd);
    else
      hipLaunchKernelGGL((skinny_mfma_kernel<TY, 4, false>), bz(grid, h->bcount), dim3(256), 0, h->stream, X, ldx, Y,
                         ldy, M, Nmax, N, K, alpha, beta, Z, ldz, out, ldo, h->bd);
  }
}

// Operand-order copy of a merge's H for the new-row and basis products: in
// the core scratch Pb (idle after the solve), past the coordinate update's
// scratch lines; none when Pb is too small or r_max > 256.
static float* merge_hf(isvd_handle* h) {
  const size_t off = 65536, need = (size_t)16 * XF_KQ * 64 * 4 * sizeof(float);
  if (h->cfg.r_max > 256 || (size_t)h->ldm * h->ldm * sizeof(double) < off + need) return nullptr;
  return (float*)((char*)h->w.Pb + off);
}

static void eig_finish(isvd_handle* h, int for_merge) {
  const isvd_ws& w = h->w;
  const int R = h->cfg.r_max;
  hipLaunchKernelGGL(eig_order_kernel, bz(dim3(1), h->bcount), dim3(1024), 0, h->stream, w.S, h->ldm, w.sig_new,
                     w.order, w.st, R, for_merge, h->bd);
  hipLaunchKernelGGL(eig_gather_kernel, bz(dim3(128), h->bcount), dim3(256), 0, h->stream, w.V, h->ldm, w.Hc, R,
                     w.order, w.st, R, for_merge, for_merge ? merge_hf(h) : nullptr, h->bd);
}

int iskv_launch_sym_eig(isvd_handle* h, const double* A, int32_t m, double* lam, double* V) {
  const isvd_ws& w = h->w;
  hipStream_t s = h->stream;
  hipLaunchKernelGGL(load_sym_kernel, dim3(128), dim3(256), 0, s, A, m, w.A, h->ldm, w.st);
  int rc = iskv_launch_core_eig(h, ISKV_EIG_TOL_EXACT);
  if (rc) return rc;
  eig_finish(h, 0);
  hipLaunchKernelGGL(store_sym_kernel, dim3(128), dim3(256), 0, s, w.S, w.V, h->ldm, w.order, m, lam, V);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

// Allow the LDS-staged update kernels to use more than 64 KB of dynamic LDS.
int iskv_kernel_setup() {
  static int done = 0;
  if (done) return ISKV_OK;
  const int lds = 160 * 1024;
  ISKV_HIP_CHECK(hipFuncSetAttribute((const void*)resid_basis_kernel<32>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)resid_lds_bytes(32)));
  const void* xh[] = {(const void*)xh_mfma_kernel<32, float, float>, (const void*)xh_mfma_kernel<16, float, float>,
                      (const void*)xh_mfma_kernel<32, uint16_t, uint16_t>,
                      (const void*)xh_mfma_kernel<16, uint16_t, uint16_t>,
                      (const void*)xh_mfma_kernel<32, float, uint16_t>,
                      (const void*)xh_mfma_kernel<16, float, uint16_t>,
                      (const void*)xh_mfma_kernel<32, _Float16, _Float16>,
                      (const void*)xh_mfma_kernel<16, _Float16, _Float16>,
                      (const void*)xh_mfma_kernel<32, float, _Float16>,
                      (const void*)xh_mfma_kernel<16, float, _Float16>,
                      (const void*)xh_mfma_kernel<16, uint16_t, float>,
                      (const void*)xh_mfma_kernel<16, _Float16, float>};
  for (const void* f : xh) ISKV_HIP_CHECK(hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds));
  if (iskv_core_eig_setup() != ISKV_OK) return ISKV_EHIP;
  done = 1;
  return ISKV_OK;
}

// The launch sequence of one merge. It depends on the host only through b
// and the handle's fixed buffers: the row count n is read on the device, so
// the sequence can be recorded once and replayed.
// Run f with the handle's coordinate array typed as stored (fp32, bf16 bits or
// IEEE half).
template <class Fn>
static void with_coords(isvd_handle* h, Fn f) {
  if (iskv_bf16_coords(h->cfg)) f((uint16_t*)h->C);
  else if (iskv_fp16_coords(h->cfg)) f((_Float16*)h->C);
  else f(h->C);
}

static int merge_body(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t b) {
  const iskv_config& c = h->cfg;
  const isvd_ws& w = h->w;
  hipStream_t s = h->stream;
  const int D = c.D, R = c.r_max;
  const int32_t* dk = w.st + ST_K;
  const int32_t* dp = w.st + ST_P;
  auto mark = [&](int i) {
    if (h->timing) (void)hipEventRecord(h->tev[i], s);
  };
  mark(0);
  // 1. Q = F B (b x k)
  skinny<false>(h, b, R, F, D, h->B, R, ddim(dk), D, 1.f, 0.f, nullptr, 0, w.Q, R);
  if (c.flags & ISKV_FROZEN_BASIS) {
    // frozen basis: the new rows keep their coordinates in B; nothing else changes
    with_coords(h, [&](auto* Cp) {
      using TC = std::remove_pointer_t<decltype(Cp)>;
      hipLaunchKernelGGL((frozen_append_kernel<TC>), bz(dim3(1), h->bcount), dim3(256), 0, s, w.Q, R, pos_F, b, Cp,
                         R, h->pos, w.st, h->bd);
    });
    for (int i = 1; i <= 5; ++i) mark(i);
    if (h->timing) h->timed = true;
    ISKV_HIP_CHECK(hipGetLastError());
    return ISKV_OK;
  }
  // 2. E = F - Q B^T (b x D)
  skinny<true>(h, b, D, w.Q, R, h->B, R, hdim(D), R, -1.f, 1.f, F, D, w.E, D);
  // 3. EB = E B; 4. E -= EB B^T (second projection, §4.1)
  skinny<false>(h, b, R, w.E, D, h->B, R, ddim(dk), D, 1.f, 0.f, nullptr, 0, w.EB, R);
  skinny<true>(h, b, D, w.EB, R, h->B, R, hdim(D), R, -1.f, 1.f, w.E, D, w.E, D);
  mark(1);
  // 5. E E^T (fp64) and the residual basis
  hipLaunchKernelGGL(resid_gram_kernel, bz(dim3(b, (b + 7) / 8), h->bcount), dim3(256), 0, s, w.E, D, b, w.GE, w.st, h->bd);
  if (b <= 32)
    hipLaunchKernelGGL(resid_basis_kernel<16>, bz(dim3(1), h->bcount), dim3(256), resid_lds_bytes(16), s, w.GE, b,
                       D, h->sigma, c.resid_rel_tol, w.VE, w.rho, w.st, ISKV_RESID_MAX_SWEEPS, h->bd);
  else
    hipLaunchKernelGGL(resid_basis_kernel<32>, bz(dim3(1), h->bcount), dim3(1024), resid_lds_bytes(32), s, w.GE, b,
                       D, h->sigma, c.resid_rel_tol, w.VE, w.rho, w.st, ISKV_RESID_MAX_SWEEPS, h->bd);
  hipLaunchKernelGGL(make_p_kernel, bz(dim3((D + 63) / 64), h->bcount), dim3(64 * ((c.b_max + 7) / 8)),
                     (size_t)(c.b_max * c.b_max + c.b_max) * sizeof(double), s, w.E, D, b, w.VE, w.rho, w.P, c.b_max,
                     w.st, h->bd);
  // 6. FP = F P (b x p)
  skinny<false>(h, b, c.b_max, F, D, w.P, c.b_max, ddim(dp), D, 1.f, 0.f, nullptr, 0, w.FP, c.b_max);
  mark(2);
  // 7. core Gram and its eigendecomposition
  {
    dim3 grid((h->m_max + 15) / 16, (h->m_max + 15) / 16);
    hipLaunchKernelGGL(core_gram_kernel, bz(grid, h->bcount), dim3(256), 0, s, w.Q, R, w.FP, c.b_max, h->sigma, b,
                       w.A, h->ldm, w.st, h->bd);
  }
  {
    int rc = iskv_launch_core_eig(h, ISKV_EIG_TOL_UPDATE, c.r_max);
    if (rc) return rc;
  }
  eig_finish(h, 1);
  const bool bf3 = c.r_max <= 256 && c.r_max % 32 == 0;  // split-bf16 coordinate update
  const int NW3 = c.r_max / 16, NS3 = c.r_max / 32;
  if (bf3 && !(c.flags & ISKV_NO_COORD_SYNC))
    // H split once into the update's operand fragments (in T2, free during a
    // merge: R / 16 x R / 32 x 64 x 2 uint4 = R^2 floats)
    hipLaunchKernelGGL(split_h_kernel, bz(dim3((NW3 * NS3 * 64 + 255) / 256), h->bcount), dim3(256), 0, s, w.Hc,
                       c.r_max, ddim(dk), ddim(w.st + ST_KNEW), NW3, NS3, (uint4*)w.T2, h->bd);
  mark(3);
  // 8. coordinate sync of old rows (n of them, read on the device), new rows
  // appended at row n, basis update
  const int M = h->m_max;
  const Dim dn = ddim(w.st + ST_N);
  with_coords(h, [&](auto* Cp) {
    using TC = std::remove_pointer_t<decltype(Cp)>;
    if (!(c.flags & ISKV_NO_COORD_SYNC)) {
      const int nblk = (c.n_cap + 15) / 16;
      const int grid = nblk < 256 ? nblk : 256;  // one workgroup per CU at most
      if (R == 256 && (size_t)c.n_cap * R * sizeof(TC) < ((size_t)1 << 31) - 4096) {
        // streaming split-bf16 update; the core scratch Pb (idle here) takes
        // the stores that nothing reads
        const int lines = (int)std::min<size_t>((size_t)h->ldm * h->ldm * 8 / 128, 256);
        hipLaunchKernelGGL((xh_bf3s_kernel<TC>), bz(dim3(grid), h->bcount), dim3(XS_NT), 0, s, Cp, R, ddim(dk),
                           (const uint4*)w.T2, NW3, NS3, ddim(w.st + ST_KNEW), dn, w.st, (float*)w.Pb, lines, h->bd);
      } else if (bf3) {  // split-bf16 matrix cores, one 1024-thread workgroup per CU at most
        hipLaunchKernelGGL((xh_bf3_kernel<TC>), bz(dim3(grid), h->bcount), dim3(1024), 0, s, Cp,
                           R, ddim(dk), (const uint4*)w.T2, NW3, NS3, ddim(w.st + ST_KNEW), dn, w.st, h->bd);
      } else {
        xh_launch(s, h->bd, h->bcount, c.n_cap, Cp, R, nullptr, 0, ddim(dk), ddim(dk), R, w.Hc, R, R,
                  ddim(w.st + ST_KNEW), dn, Cp, R, nullptr, 0, nullptr, nullptr, false, hdim(0), w.st);
      }
    }
    mark(4);
    const float4* Hf = (const float4*)merge_hf(h);
    if (std::is_same<TC, float>::value && M <= 288 && R <= 256) {
      // new rows and basis update in one launch (both read H in operand order)
      const int gn = (b + 15) / 16, gd = std::min((D + 15) / 16, 256);
      const XhJob<float, float> A = {w.Q, R, w.FP, c.b_max, ddim(dk), ddim(w.st + ST_M), w.Hc, R, R,
                                     ddim(w.st + ST_KNEW), hdim(b), (float*)Cp, R, nullptr, 0, h->pos, pos_F, dn,
                                     Hf, gn};
      const XhJob<float, float> Bj = {h->B, R, w.P, c.b_max, ddim(dk), ddim(w.st + ST_M), w.Hc, R, R,
                                      ddim(w.st + ST_KNEW), hdim(D), h->B, R, w.Bbf, R, nullptr, nullptr, hdim(0),
                                      Hf, gd};
      if (M <= 256)
        hipLaunchKernelGGL((xh_reg2_kernel<64, float, float>), bz(dim3(gn + gd), h->bcount), dim3(1024), 0, s, A, Bj,
                           w.st, h->bd);
      else
        hipLaunchKernelGGL((xh_reg2_kernel<72, float, float>), bz(dim3(gn + gd), h->bcount), dim3(1024), 0, s, A, Bj,
                           w.st, h->bd);
    } else {
      xh_launch(s, h->bd, h->bcount, b, w.Q, R, w.FP, c.b_max, ddim(dk), ddim(w.st + ST_M), M, w.Hc, R, R,
                ddim(w.st + ST_KNEW), hdim(b), Cp, R, nullptr, 0, h->pos, pos_F, false, dn, w.st, Hf);
      xh_launch(s, h->bd, h->bcount, D, h->B, R, w.P, c.b_max, ddim(dk), ddim(w.st + ST_M), M, w.Hc, R, R,
                ddim(w.st + ST_KNEW), hdim(D), h->B, R, w.Bbf, R, nullptr, nullptr, true, hdim(0), nullptr, Hf);
    }
  });
  hipLaunchKernelGGL(merge_commit_kernel, bz(dim3(1), h->bcount), dim3(256), 0, s, h->sigma, w.sig_new, w.st, b, R, h->bd);
  mark(5);
  if (h->timing) h->timed = true;
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

// Re-orthogonalisation (iS-KV notes §4.4), written with Grams instead of the
// notes' thin QRs: with G_B = B^T B = M_B^2 (M_B its symmetric square root,
// Z = M_B^-1 by Newton-Schulz) and G_C = C^T C, the eigendecomposition
// M_B G_C M_B = Y Lambda Y^T gives C' = C M_B Y (orthogonal columns, norms
// sqrt(Lambda)) and B' = B Z Y (orthonormal), with C' B'^T = C B^T. This is
// the notes' U <- Q_U W, B <- Q_B V with R_U Sigma R_B^T = W S V^T expressed
// through M = R_U Sigma R_B^T's right singular vectors.
// Launch sequence of one re-orthogonalisation; the row count n is read on
// the device (chunks of C beyond n contribute zero Grams).
static int reorth_body(isvd_handle* h) {
  const iskv_config& c = h->cfg;
  const isvd_ws& w = h->w;
  hipStream_t s = h->stream;
  const int R = c.r_max, D = c.D, mm = h->m_max, ld = h->ldm;
  const int ncap = c.n_cap;
  const int tiles = (R + 15) / 16;
  const int rows_per_chunk = 1024;
  int nchunks = (ncap + rows_per_chunk - 1) / rows_per_chunk;
  if (nchunks > w.gram_splits - 1) nchunks = w.gram_splits - 1;
  const int rpc = (ncap + nchunks - 1) / nchunks;
  const Dim dn = ddim(w.st + ST_N);
  hipLaunchKernelGGL(set_jm_kernel, bz(dim3(1), h->bcount), dim3(1), 0, s, w.st, (int)ST_K, h->bd);
  with_coords(h, [&](auto* Cp) {
    using TC = std::remove_pointer_t<decltype(Cp)>;
    hipLaunchKernelGGL((gram_partial_kernel<TC>), bz(dim3(tiles * tiles, nchunks), h->bcount), dim3(256), 0, s,
                       (const TC*)Cp, R, dn, w.st, w.GC, R, rpc, h->bd);
  });
  hipLaunchKernelGGL(gram_partial_kernel<float>, bz(dim3(tiles * tiles, 1), h->bcount), dim3(256), 0, s, h->B, R, hdim(D), w.st,
                     w.GC + (size_t)nchunks * R * R, R, D, h->bd);
  hipLaunchKernelGGL(reorth_sum_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.GC, nchunks, R, w.Km, w.Pa, w.Pb,
                     ld, w.st, h->bd);
  const int32_t* st = w.st;
  // Z = Z0 (3I - G_B Z0^2) / 2 = 1.5 Z0 - 0.5 Z0 (G_B Z0 Z0)   (second Newton-Schulz step)
  iskv_dgemm(s, mm, w.Pa, false, w.Pb, false, w.T, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  iskv_dgemm(s, mm, w.T, false, w.Pb, false, w.S, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  iskv_dgemm(s, mm, w.Pb, false, w.S, false, w.Zb, w.Pb, ld, -0.5, 1.5, 0.0, st, 2, h->bd, h->bcount);
  // M_B = G_B Z;  H = M_B G_C M_B^T -> A
  iskv_dgemm(s, mm, w.Pa, false, w.Zb, false, w.MB, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  iskv_dgemm(s, mm, w.MB, false, w.Km, false, w.T, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  iskv_dgemm(s, mm, w.T, false, w.MB, true, w.A, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  {
    int rc = iskv_launch_core_eig(h, ISKV_EIG_TOL_UPDATE, ISKV_EIG_KEEP_ALL);
    if (rc) return rc;
  }
  eig_finish(h, 0);
  hipLaunchKernelGGL(permute_cols_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.V, w.order, w.W1, ld, w.st, h->bd);
  // T1 = M_B^T Y (coordinates), T2 = Z Y (basis)
  iskv_dgemm(s, mm, w.MB, true, w.W1, false, w.T, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  iskv_dgemm(s, mm, w.Zb, false, w.W1, false, w.Pa, nullptr, ld, 1.0, 0.0, 0.0, st, 2, h->bd, h->bcount);
  hipLaunchKernelGGL(to_f32_kernel, bz(dim3(128), h->bcount), dim3(256), 0, s, w.T, w.Pa, ld, w.Hc, w.T2, R, w.st, h->bd);
  with_coords(h, [&](auto* Cp) {
    xh_launch(s, h->bd, h->bcount, ncap, Cp, R, nullptr, 0, ddim(w.st + ST_K), ddim(w.st + ST_K), R, w.Hc, R, R,
              ddim(w.st + ST_K), dn, Cp, R, nullptr, 0, nullptr, nullptr, false, hdim(0), w.st);
  });
  xh_launch(s, h->bd, h->bcount, D, h->B, R, nullptr, 0, ddim(w.st + ST_K), ddim(w.st + ST_K), R, w.T2, R, R,
            ddim(w.st + ST_K), hdim(D), h->B, R, w.Bbf, R, nullptr, nullptr, true);
  hipLaunchKernelGGL(reorth_commit_kernel, bz(dim3(1), h->bcount), dim3(256), 0, s, h->sigma, w.sig_new, w.st, R, h->bd);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

namespace {

// Stage the pending blocks of a batch: copy z takes block z of the caller's
// arrays (F + z F_stride, pos_F + z pos_stride) into its handle's workspace.
__global__ void stage_batch_kernel(const float* __restrict__ F, int64_t F_stride,
                                   const int32_t* __restrict__ pos_F, int64_t pos_stride, float* Fs,
                                   int32_t* posFs, int count, int b, const int64_t* __restrict__ bd) {
  const int z = blockIdx.z;
  const int64_t d = bd[z];
  Fs = iskv_rb(Fs, d);
  posFs = iskv_rb(posFs, d);
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) Fs[i] = F[z * F_stride + i];
  if (i < b) posFs[i] = pos_F[z * pos_stride + i];
}

// Stage a pending block in the workspace (the recorded merge reads it there).
__global__ void stage_block_kernel(const float* __restrict__ F, const int32_t* __restrict__ pos_F,
                                   float* Fs, int32_t* posFs, int count, int b) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) Fs[i] = F[i];
  if (i < b) posFs[i] = pos_F[i];
}

bool use_graphs(const isvd_handle* h) {
  return h->stream != nullptr && !(h->cfg.flags & ISKV_NO_GRAPH) && !h->timing;
}

// Record `body` on the handle's stream into an executable graph.
template <class Body>
int record(isvd_handle* h, hipGraphExec_t* exec, Body body) {
  hipGraph_t g = nullptr;
  ISKV_HIP_CHECK(hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
  const int rc = body();
  const hipError_t ec = hipStreamEndCapture(h->stream, &g);
  if (rc != ISKV_OK) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (ec != hipSuccess || !g) return ISKV_EHIP;
  const hipError_t ei = hipGraphInstantiate(exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (ei != hipSuccess) {
    *exec = nullptr;
    return ISKV_EHIP;
  }
  return ISKV_OK;
}

}  // namespace

void iskv_release_graphs(isvd_handle* h) {
  if (h->g_merge) (void)hipGraphExecDestroy(h->g_merge);
  if (h->g_reorth) (void)hipGraphExecDestroy(h->g_reorth);
  if (h->g_batch_merge) (void)hipGraphExecDestroy(h->g_batch_merge);
  if (h->g_batch_reorth) (void)hipGraphExecDestroy(h->g_batch_reorth);
  h->g_merge = nullptr;
  h->g_reorth = nullptr;
  h->g_batch_merge = nullptr;
  h->g_batch_reorth = nullptr;
  h->g_batch_set.clear();
}

// One merge. Without graphs the sequence is enqueued directly. With graphs,
// the sequence recorded for (b, block pointers) is replayed; a caller whose
// block pointers change between calls gets its block staged in the workspace
// and a sequence recorded once over the staged copy.
int iskv_launch_merge(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t b) {
  if (!use_graphs(h)) return merge_body(h, F, pos_F, b);
  const bool same = h->g_merge && h->g_merge_b == b && h->g_merge_F == F && h->g_merge_posF == pos_F;
  if (!same) {
    const float* gF = F;
    const int32_t* gP = pos_F;
    if (h->g_merge && h->g_merge_b == b && h->g_merge_F == h->w.Fs) {
      gF = h->w.Fs;
      gP = h->w.posFs;
    } else if (h->g_merge) {
      // pointers or b changed since the last recording: record over the
      // staged copy from now on
      gF = h->w.Fs;
      gP = h->w.posFs;
      (void)hipGraphExecDestroy(h->g_merge);
      h->g_merge = nullptr;
    }
    if (gF == h->w.Fs) {
      const int count = b * h->cfg.D;
      hipLaunchKernelGGL(stage_block_kernel, dim3((count + 255) / 256), dim3(256), 0, h->stream, F, pos_F,
                         h->w.Fs, h->w.posFs, count, b);
      ISKV_HIP_CHECK(hipGetLastError());
    }
    if (!h->g_merge) {
      int rc = record(h, &h->g_merge, [&]() { return merge_body(h, gF, gP, b); });
      if (rc) return rc;
      h->g_merge_b = b;
      h->g_merge_F = gF;
      h->g_merge_posF = gP;
    }
  }
  ISKV_HIP_CHECK(hipGraphLaunch(h->g_merge, h->stream));
  return ISKV_OK;
}

int iskv_launch_reorth(isvd_handle* h) {
  if (h->n_host == 0) return ISKV_OK;
  if (!use_graphs(h)) return reorth_body(h);
  if (!h->g_reorth) {
    int rc = record(h, &h->g_reorth, [&]() { return reorth_body(h); });
    if (rc) return rc;
  }
  ISKV_HIP_CHECK(hipGraphLaunch(h->g_reorth, h->stream));
  return ISKV_OK;
}

// ---------------------------------------------------------------------------
// Fresh truncated SVD of given rows (Algorithm 1, the value first
// refit of §3.2): after the rows are folded by merges, subspace iterations
// with a Rayleigh-Ritz step converge to the top-k right singular subspace of X.
// Each iteration:
//   C <- X B and re-orthogonalise (§4.4): with B orthonormal, C B^T = X B B^T
//     becomes its exact SVD, whose right singular vectors are the Ritz
//     vectors of X^T X in span(B) and whose coordinates are X B;
//   Z <- X^T C (= X^T X B);  B <- Z diag(1 / |z_j|), orthonormalised by
//   shifted CholeskyQR3 (the first pass shifted, so that a numerically
//   rank-deficient Z in fp32 stays factorable with bounded growth).
// A last Ritz step gives the factors C = X B. The Ritz cores can be dense;
// their eigensolves take the block Jacobi fallback.
namespace {

// Bt[j][d] = B[d][j] (32 x 32 tiles through LDS).
__global__ __launch_bounds__(256) void transpose_b_kernel(const float* __restrict__ B, int D, int R,
                                                          float* __restrict__ Bt) {
  __shared__ float tile[32][33];
  const int d0 = blockIdx.x * 32, j0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int yy = ty; yy < 32; yy += 8)
    tile[yy][tx] = (d0 + yy < D && j0 + tx < R) ? B[(size_t)(d0 + yy) * R + j0 + tx] : 0.f;
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8)
    if (j0 + yy < R && d0 + tx < D) Bt[(size_t)(j0 + yy) * D + d0 + tx] = tile[tx][yy];
}

}  // namespace

// Y (n x D, fp32, path order) = C B^T: the rows the history represents.
int iskv_launch_materialize(isvd_handle* h, float* Y, float* Bt) {
  const iskv_config& c = h->cfg;
  hipStream_t s = h->stream;
  const int D = c.D, R = c.r_max, n = h->n_host;
  if (n == 0) return ISKV_OK;
  if (xh_lds_bytes(16, R) > 160 * 1024) return ISKV_EINVAL;
  hipLaunchKernelGGL(transpose_b_kernel, dim3((D + 31) / 32, (R + 31) / 32), dim3(256), 0, s, h->B, D, R, Bt);
  with_coords(h, [&](auto* Cp) {
    xh_launch(s, nullptr, 1, n, Cp, R, nullptr, 0, ddim(h->w.st + ST_K), ddim(h->w.st + ST_K), R, Bt, D, D, hdim(D),
              hdim(n), Y, D, nullptr, 0, nullptr, nullptr, true);
  });
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

// C <- X B stages 16 rows of X (D wide) in LDS: D up to 1984.
bool iskv_refit_supported(const iskv_config& c) { return xh_lds_bytes(16, c.D) <= 160 * 1024; }

size_t iskv_refit_ws_bytes(const isvd_handle* h) { return iskv_refit_gram_ws_bytes(h); }

// C <- X B over the n rows X (n x D fp32), k = st[ST_K] columns; stored as
// the handle keeps its coordinates (fp32, bf16 or fp16).
int iskv_launch_coords_from_rows(isvd_handle* h, const float* X, int32_t n) {
  const iskv_config& c = h->cfg;
  const int D = c.D, R = c.r_max;
  with_coords(h, [&](auto* Cp) {
    xh_launch(h->stream, nullptr, 1, n, X, D, nullptr, 0, hdim(D), hdim(D), D, h->B, R, R, ddim(h->w.st + ST_K),
              hdim(n), Cp, R, nullptr, 0, nullptr, nullptr, true, hdim(0), h->w.st);
  });
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

// ---------------------------------------------------------------------------
// Batched merges / reorths over handles with one configuration and one buffer
// layout (every buffer of handle z lies at the same byte offset from the
// corresponding buffer of handle 0; checked by the caller): the launch
// sequence of one merge runs once with grid.z = count and each copy rebased
// by its handle's offset. The offsets live in the first handle's workspace.
int iskv_upload_offsets(isvd_handle* const* hs, int32_t count) {
  isvd_handle* h0 = hs[0];
  if ((int)h0->g_batch_set.size() == count &&
      std::equal(h0->g_batch_set.begin(), h0->g_batch_set.end(), hs))
    return ISKV_OK;
  // a new set of handles: new offsets, and the recorded sequences are stale
  if (h0->g_batch_merge) (void)hipGraphExecDestroy(h0->g_batch_merge);
  if (h0->g_batch_reorth) (void)hipGraphExecDestroy(h0->g_batch_reorth);
  h0->g_batch_merge = nullptr;
  h0->g_batch_reorth = nullptr;
  std::vector<int64_t> off(count);
  for (int z = 0; z < count; ++z) off[z] = (const char*)hs[z]->ws_base - (const char*)h0->ws_base;
  ISKV_HIP_CHECK(hipMemcpyAsync(h0->w.btab, off.data(), count * sizeof(int64_t), hipMemcpyHostToDevice,
                                h0->stream));
  ISKV_HIP_CHECK(hipStreamSynchronize(h0->stream));  // `off` is released on return
  h0->g_batch_set.assign(hs, hs + count);
  return ISKV_OK;
}

namespace {

template <class Body>
int run_batched(isvd_handle* h0, int32_t count, hipGraphExec_t* cache, Body body) {
  h0->bd = h0->w.btab;
  h0->bcount = count;
  int rc = ISKV_OK;
  if (!use_graphs(h0)) {
    rc = body();
  } else {
    if (!*cache) rc = record(h0, cache, body);
    if (rc == ISKV_OK && hipGraphLaunch(*cache, h0->stream) != hipSuccess) rc = ISKV_EHIP;
  }
  h0->bd = nullptr;
  h0->bcount = 1;
  return rc;
}

}  // namespace

int iskv_launch_merge_batched(isvd_handle* const* hs, int32_t count, const float* F, int64_t F_stride,
                              const int32_t* pos_F, int64_t pos_stride, int32_t b) {
  isvd_handle* h0 = hs[0];
  int rc = iskv_upload_offsets(hs, count);
  if (rc) return rc;
  if (h0->g_batch_merge && h0->g_batch_b != b) {
    (void)hipGraphExecDestroy(h0->g_batch_merge);
    h0->g_batch_merge = nullptr;
  }
  const int n = b * h0->cfg.D;
  hipLaunchKernelGGL(stage_batch_kernel, dim3((n + 255) / 256, 1, count), dim3(256), 0, h0->stream, F, F_stride,
                     pos_F, pos_stride, h0->w.Fs, h0->w.posFs, n, b, (const int64_t*)h0->w.btab);
  ISKV_HIP_CHECK(hipGetLastError());
  rc = run_batched(h0, count, &h0->g_batch_merge,
                   [&]() { return merge_body(h0, h0->w.Fs, h0->w.posFs, b); });
  if (rc == ISKV_OK) h0->g_batch_b = b;
  return rc;
}

int iskv_launch_reorth_batched(isvd_handle* const* hs, int32_t count) {
  isvd_handle* h0 = hs[0];
  int rc = iskv_upload_offsets(hs, count);
  if (rc) return rc;
  return run_batched(h0, count, &h0->g_batch_reorth, [&]() { return reorth_body(h0); });
}
