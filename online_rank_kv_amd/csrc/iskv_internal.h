// Internal declarations of the gfx950 iS-KV library: handle layout, device
// state slots and the launch helpers shared by the translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/iskv.h"

#include <type_traits>
#include <vector>

// ---- device state word slots (int32 array at the head of the workspace) ----
enum {
  ST_N = 0,        // rows in the compressed history
  ST_K = 1,        // current rank k
  ST_P = 2,        // residual directions kept by the last merge
  ST_FOLDED = 3,   // regular folded rows (re-orthogonalisation schedule)
  ST_STATUS = 4,   // ISKV_DEV_* bits
  ST_M = 5,        // core width k + p of the merge in flight
  ST_KNEW = 6,     // r' = min(r, k + p) of the merge in flight
  ST_SWEEPS = 7,   // Jacobi sweeps used by the last eigensolve
  ST_EZERO = 8,    // 1 when the residual of the merge in flight is exactly zero
  ST_JM = 9,       // order of the matrix handed to the Jacobi eigensolver
  ST_ROUNDS = 10,  // 1 when the refinement's W failed its orthogonality check (cold fallback)
  ST_PCJ = 11,     // core eigensolver flags: 1 converged, 2 Jacobi fallback used
  ST_PCJIT = 12,   // refinement steps used by the last core eigensolve
  ST_NEDGE = 13,   // strong pairs found by the current detection pass
  ST_RSWEEPS = 14, // Jacobi sweeps of the last residual eigensolve
  ST_SREF = 15,    // core eigensolver: fp32 bits of max_i A_ii (coupling scale), 0 = scaled couplings
  ST_DCUT = 16,    // core eigensolver: fp32 bits of the diagonal value between kept and dropped, < 0 = none
  ST_NROT = 17,    // core eigensolver: exact rotation groups of the refinement step in flight
  ST_COUNT = 20
};

// Sub-buffers carved out of the caller's workspace (all 256-byte aligned).
struct isvd_ws {
  int32_t* st;        // [ST_COUNT]
  uint16_t* Bbf;      // [D x r_max] bf16 copy of B for reconstruction
  float* Q;           // [b_max x r_max]  F B
  float* E;           // [b_max x D]      residual
  float* EB;          // [b_max x r_max]  E B
  double* GE;         // [b_max x b_max]  E E^T
  double* VE;         // [b_max x b_max]  its eigenvectors (sorted)
  double* rho;        // [b_max]          residual singular values
  float* P;           // [D x b_max]      residual basis
  float* FP;          // [b_max x b_max]  F P
  double* A;          // [ldm x ldm]  core Gram / reorth matrix
  double* V;          // [ldm x ldm]  eigenvectors
  double* S;          // [ldm x ldm]  W^T A W / Jacobi working matrix
  double* W0;         // [ldm x ldm]  eigenvector iterate (ping)
  double* W1;         // [ldm x ldm]  eigenvector iterate (pong)
  double* T;          // [ldm x ldm]  A W
  double* Km;         // [ldm x ldm]  first-order angles K
  double* Pa;         // [ldm x ldm]  exp(K) partial products
  double* Pb;         // [ldm x ldm]
  double* MB;         // [ldm x ldm]  reorth: (B^T B)^(1/2)
  double* Zb;         // [ldm x ldm]  reorth: (B^T B)^(-1/2)
  double* aux;        // [naux] per-tile / per-block maxima of the scaled coupling
  int32_t* edges;     // [ISKV_PCJ_EMAX x 2] strongly coupled pairs of a refinement step
  int32_t* itab;      // refinement step's exact rotations: group of each index, its place, group sizes, members
  double* rtab;       // their rotated diagonal [m_max] and rotation matrices [groups x ISKV_PCJ_CMAX^2]
  double* Dp;         // [ldm / 16 x ldm] partial sums of diag(W^T A W) per 16-row block
  double* lam;        // [m_max]
  double* rot;        // [rot_cap] Jacobi rotation log (c, s) pairs
  float* Hc;          // [m_max x r_max]  kept right singular vectors of the core
  float* T2;          // [r_max x r_max]  second transform (reorth: basis side)
  float* sig_new;     // [m_max]
  double* GC;         // [gram_splits x r_max x r_max] partial Grams for reorth
  double* GB;         // [r_max x r_max]
  double* RB;         // [r_max x r_max]  Cholesky factor of B^T B
  int32_t* order;     // [m_max]
  float* Fs;          // [b_max x D]  staged pending block (graph replays read it)
  int32_t* posFs;     // [b_max]      its positions
  int64_t* btab;      // [ISKV_MAX_BATCH] per-handle byte offsets of a batched launch
  size_t rot_cap;     // doubles in rot
  int naux;           // doubles in aux
  int gram_splits;
};

// stage boundaries of a merge recorded by isvd_set_timing
#define ISKV_STAGES 5

struct isvd_handle {
  iskv_config cfg;
  float* C;
  float* sigma;
  float* B;
  int32_t* pos;
  void* ws_base;
  size_t ws_bytes;
  hipStream_t stream;
  isvd_ws w;
  int32_t m_max;       // r_max + b_max
  int32_t ldm;         // leading dimension of the fp64 core matrices
  int32_t n_host;      // rows folded (host mirror, exact)
  int32_t folded_host; // folded-row counter (host mirror, exact)
  // recorded launch sequences (HIP graphs) of a merge and of a reorth
  hipGraphExec_t g_merge = nullptr;
  int32_t g_merge_b = 0;
  const float* g_merge_F = nullptr;      // block pointers the merge graph reads
  const int32_t* g_merge_posF = nullptr;
  hipGraphExec_t g_reorth = nullptr;
  // batched launches: every merge / reorth kernel runs grid.z = bcount copies,
  // copy z rebasing each pointer it is given by bd[z] bytes (bd = nullptr for
  // one handle); set only while a batched launch sequence is enqueued
  const int64_t* bd = nullptr;
  int32_t bcount = 1;
  // recorded batched merge / reorth (kept by the first handle of the batch)
  std::vector<isvd_handle*> g_batch_set;
  int32_t g_batch_b = 0;
  hipGraphExec_t g_batch_merge = nullptr;
  hipGraphExec_t g_batch_reorth = nullptr;
  // stage timing (isvd_set_timing): merges run eager with an event at every
  // stage boundary
  bool timing = false;
  bool timed = false;  // a merge has been timed since timing was switched on
  hipEvent_t tev[ISKV_STAGES + 1] = {};
  // the next core eigensolve is of a dense matrix: straight to the block
  // Jacobi, no refinement (set around eager solves of the refit's
  // Rayleigh-Ritz core, never while recording)
  bool force_block_jacobi = false;
};

struct iskv_window {
  isvd_handle* h;
  int32_t D, prot_cap, window, block;
  float* rows;
  int32_t* pos;
  hipStream_t stream;
  int32_t n_prot;      // protected rows stored
  int64_t appended;    // rows appended through the window
  int32_t pending;     // rows waiting in the pending area
  int32_t prot_flags;  // unused, reserved
};

#define ISKV_JACOBI_MAX_SWEEPS 40
// Strongly coupled pairs recorded per refinement step of the core solver.
#define ISKV_PCJ_EMAX 4096
#define ISKV_PCJ_CMAX 6   // largest cluster the refinement diagonalises exactly
// K-panel depth of the fp64 core GEMM; the leading dimension of every fp64
// core matrix in the workspace is a multiple of it.
#define ISKV_DGEMM_KP 288
// Largest number of handles one batched merge may serve.
#define ISKV_MAX_BATCH 4096
inline int iskv_core_ld(int m_max) { return (m_max + ISKV_DGEMM_KP - 1) / ISKV_DGEMM_KP * ISKV_DGEMM_KP; }
#define ISKV_RESID_MAX_SWEEPS 30

// ---- launch helpers implemented in the kernel translation units ----
int iskv_kernel_setup();
int iskv_core_eig_setup();
// Core eigensolver on w.A; stops when every coupling is below tol: the
// scaled coupling (every eigenvector to tol) when keep < 0, else the
// coupling's effect on the represented product (merges keep = r_max, the
// re-orthogonalisation keeps everything: ISKV_EIG_KEEP_ALL).
constexpr int ISKV_EIG_SCALED = -1;
constexpr int ISKV_EIG_KEEP_ALL = 0x7fffffff;
int iskv_launch_core_eig(isvd_handle* h, double tol, int keep = ISKV_EIG_SCALED);
#define ISKV_EIG_TOL_EXACT 1e-10   // isvd_sym_eig
#define ISKV_EIG_TOL_UPDATE 1e-8   // merges and re-orthogonalisations
void iskv_dgemm(hipStream_t s, int m_max, const double* A, bool ta, const double* B, bool tb, double* C,
                const double* Cin, int ld, double alpha, double beta, double gamma, const int32_t* st,
                int mode, const int64_t* bd, int bc);
int iskv_launch_merge(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t b);
int iskv_launch_merge_batched(isvd_handle* const* hs, int32_t count, const float* F, int64_t F_stride,
                              const int32_t* pos_F, int64_t pos_stride, int32_t b);
int iskv_launch_reorth_batched(isvd_handle* const* hs, int32_t count);
int iskv_launch_reorth(isvd_handle* h);
void iskv_release_graphs(isvd_handle* h);
int iskv_launch_sym_eig(isvd_handle* h, const double* A, int32_t m, double* lam, double* V);
bool iskv_recon_stream_ok(const isvd_handle* h, int32_t n_total, int32_t head_dim);
int iskv_launch_reconstruct_batched(const isvd_handle* const* hs, int32_t count, uint16_t* const* outs,
                                    const int32_t* n_totals, const int32_t* ropes, int32_t head_dim,
                                    float rope_theta, hipStream_t s, const float* X_exact,
                                    const int32_t* pos_exact, int32_t n_exact);
int iskv_launch_exact_rows(const float* X_exact, const int32_t* pos_exact, int32_t n_exact, int32_t D,
                           int32_t n_total, int32_t head_dim, int32_t apply_rope, float rope_theta,
                           void* out, int32_t out_dtype, hipStream_t s);
int iskv_launch_reconstruct(const isvd_handle* h, const float* X_exact, const int32_t* pos_exact,
                            int32_t n_exact, int32_t n_total, int32_t head_dim, int32_t apply_rope,
                            float rope_theta, void* out, int32_t out_dtype, hipStream_t s);
int iskv_launch_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch,
                       int32_t n, int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out,
                       void* ws, size_t ws_bytes, hipStream_t s);
size_t iskv_attend_ws_bytes(int32_t batch, int32_t n, int32_t Hq, int32_t dh);
// decode attention with its partials in the library's fixed device scratch
int iskv_launch_attend_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch, int32_t n,
                               int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out, hipStream_t s);
size_t iskv_attend_fv_ws_bytes(int32_t n_c, int32_t n_exact, int32_t Hq, int32_t r_max);
int iskv_launch_attend_fv(const uint16_t* q, const uint16_t* K, const isvd_handle* hv, const float* X_exact,
                          const int32_t* pos_exact, int32_t n_exact, int32_t n_total, int32_t Hq, int32_t Hkv,
                          float scale, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s);
bool iskv_refit_supported(const iskv_config& c);
size_t iskv_refit_ws_bytes(const isvd_handle* h);
// Fresh truncated SVD of n rows (refit_gram.hip): subspace block width, its
// workspace, and the launch sequence (iters subspace iterations, >= 1).
int iskv_refit_block(const isvd_handle* h);
size_t iskv_refit_gram_ws_bytes(const isvd_handle* h);
int iskv_launch_refit_gram(isvd_handle* h, const float* X, int32_t n, int32_t iters, void* work);
// C <- X B for the n rows X (n x D fp32), k = st[ST_K] columns.
int iskv_launch_coords_from_rows(isvd_handle* h, const float* X, int32_t n);
int iskv_launch_materialize(isvd_handle* h, float* Y, float* Bt);
size_t iskv_prompt_split_ws_bytes(int32_t L);
int iskv_launch_prompt_split(const float* X, const uint8_t* flags, int32_t L, int32_t D, uint32_t mask, int32_t pos0,
                             float* X_keep, int32_t* pos_keep, float* X_rest, int32_t* pos_rest, int32_t* counts,
                             void* ws, hipStream_t s);
size_t iskv_prompt_protect_ws_bytes(int32_t L, int32_t Hkv, int32_t block, int32_t suffix_blocks);
int iskv_launch_prompt_protect(const uint16_t* K_rot, int32_t L, int32_t Hkv, int32_t dh, int32_t block,
                               int32_t per_head, int32_t suffix_blocks, int32_t v_radius, int32_t v_window,
                               uint8_t* flags, float* scores_out, void* ws, size_t ws_bytes, hipStream_t s);
// Window row moves and position fills; with bd (count bc) every copy z is
// rebased by bd[z] bytes (see move_rows_kernel).
int iskv_launch_window_move(float* dst_rows, int32_t* dst_pos, const float* src_rows,
                            const int32_t* src_pos, int32_t src_pos_base, int32_t count, int32_t D,
                            hipStream_t s, const int64_t* bd = nullptr, int32_t bc = 1,
                            int32_t src_rebased = 1, int64_t src_stride = 0);
int iskv_launch_fill_pos(int32_t* pos, int32_t count, int32_t value0, int32_t step, hipStream_t s,
                         const int64_t* bd = nullptr, int32_t bc = 1);
// Upload the byte offsets of handles hs[1..] from hs[0] (workspace bases) to
// hs[0]'s offset table; no-op when the same set was uploaded last.
int iskv_upload_offsets(isvd_handle* const* hs, int32_t count);
int iskv_launch_copy_pos_host(int32_t* pos_dev, const int32_t* pos_host, int32_t count,
                              hipStream_t s);

// Stored coordinates: fp32, bf16 (uint16 bits) under ISKV_BF16_COORDS, or
// IEEE half (_Float16) under ISKV_FP16_COORDS. Loads widen to fp32; stores
// round to nearest even (NaN stays NaN) and return whether the value had to
// be saturated: only the half store can, at magnitudes above 65504 (its
// largest finite value), where it writes +-65504 instead of an infinity.
// Kernels OR the returned flags and latch ISKV_DEV_FP16_OVERFLOW once.
__device__ __forceinline__ float iskv_ld(const float* p) { return *p; }
__device__ __forceinline__ float iskv_ld(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float iskv_ld(const _Float16* p) { return (float)*p; }
__device__ __forceinline__ uint16_t iskv_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
constexpr float ISKV_F16_MAX = 65504.f;
__device__ __forceinline__ bool iskv_f16_over(float v) { return fabsf(v) > ISKV_F16_MAX; }  // NaN: false
__device__ __forceinline__ _Float16 iskv_to_f16(float v) {
  return (_Float16)(iskv_f16_over(v) ? copysignf(ISKV_F16_MAX, v) : v);
}
__device__ __forceinline__ bool iskv_st(float* p, float v) { *p = v; return false; }
__device__ __forceinline__ bool iskv_st(uint16_t* p, float v) { *p = iskv_to_bf16(v); return false; }
__device__ __forceinline__ bool iskv_st(_Float16* p, float v) {
  *p = iskv_to_f16(v);
  return iskv_f16_over(v);
}
template <class TC>
__device__ __forceinline__ void iskv_latch_overflow(int32_t* st, bool over) {
  if constexpr (sizeof(TC) == 2 && !std::is_same<TC, uint16_t>::value)
    if (over) atomicOr(&st[ST_STATUS], ISKV_DEV_FP16_OVERFLOW);
}
inline bool iskv_bf16_coords(const iskv_config& c) { return (c.flags & ISKV_BF16_COORDS) != 0; }
inline bool iskv_fp16_coords(const iskv_config& c) { return (c.flags & ISKV_FP16_COORDS) != 0; }
// bytes per stored coordinate
inline int iskv_coord_bytes(const iskv_config& c) { return (c.flags & (ISKV_BF16_COORDS | ISKV_FP16_COORDS)) ? 2 : 4; }

// Batched launches: z copies of a grid, and the per-copy pointer rebase.
inline dim3 bz(dim3 g, int count) { return dim3(g.x, g.y, (unsigned)count); }
template <class T>
__device__ __forceinline__ T* iskv_rb(T* p, int64_t d) {
  return p ? (T*)((const char*)p + d) : p;
}

#define ISKV_HIP_CHECK(expr)                 \
  do {                                       \
    hipError_t _e = (expr);                  \
    if (_e != hipSuccess) return ISKV_EHIP;  \
  } while (0)
