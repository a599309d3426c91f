/*
 * iskv.h - C ABI of the MI355X (gfx950) hot path of iS-KV online low-rank KV
 * compression: block-incremental SVD merges of pending exact KV blocks into a
 * truncated history, periodic re-orthogonalisation, reconstruction of the
 * dense cache with per-position RoPE, and GQA decode attention over it.
 *
 * Source of the method: Zhongzhu Zhou, reading notes on "iS-KV: Online
 * Low-Rank KV Cache Compression via Block-Incremental SVD" ("iS-KV notes"
 * below), sections 2-5, Algorithms 1-3, eq.(3), eq.(7), eq.(12).
 *
 * Conventions shared by every entry point
 *  - Plain C: no C++ or torch types cross this boundary. Device buffers are
 *    plain device pointers; streams are hipStream_t passed as void*
 *    (NULL = the null stream).
 *  - Ownership: the caller allocates and owns every device buffer (factors,
 *    positions, workspace, outputs). The library never allocates device
 *    memory; it only malloc()s the small host-side handle objects.
 *  - Asynchrony: every call only enqueues kernels on the handle's stream and
 *    returns without waiting, except isvd_query(), which synchronises that
 *    stream to read the device-side counters.
 *  - Errors: 0 on success, a negative ISKV_E* code otherwise. Arguments are
 *    checked before anything is enqueued, and a call that fails its checks
 *    leaves every buffer and the handle unchanged. Numerical trouble found on
 *    the device (non-finite input, a core eigensolver that did not converge)
 *    is latched in the device status word and reported by isvd_query(); the
 *    kernels never index memory with data-derived values that such input could
 *    corrupt. No C++ exception crosses the ABI.
 *  - Threading: a handle is not thread-safe; drive it from one host thread
 *    and one stream.
 *  - Layouts are row-major. Floating point is IEEE fp32 unless stated;
 *    bf16 values are passed as their uint16_t bit patterns.
 */
#ifndef ISKV_H
#define ISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum iskv_status {
  ISKV_OK = 0,
  ISKV_EINVAL = -1,      /* bad shape, null pointer, inconsistent argument     */
  ISKV_ECAPACITY = -2,   /* n + b would exceed n_cap, or a window is full      */
  ISKV_EWORKSPACE = -3,  /* workspace too small or misaligned                  */
  ISKV_EHIP = -4,        /* a HIP runtime call failed                          */
  ISKV_ENONFINITE = -5,  /* a merged block or the core held NaN/Inf (latched)  */
  ISKV_ENOCONV = -6,     /* the core eigensolver hit its sweep cap (latched)   */
  ISKV_EMODE = -7        /* operation not available in this handle's mode      */
};

/* Device status word bits (isvd_query's *status). */
#define ISKV_DEV_NONFINITE 1
#define ISKV_DEV_NOCONV 2
#define ISKV_DEV_FP16_OVERFLOW 4 /* under ISKV_FP16_COORDS: a coordinate written
                                    to the fp16 store had magnitude above 65504,
                                    the largest finite fp16 (iS-KV notes §7.3:
                                    derived factors, whose scale carries the
                                    singular values, can pass it while the K/V
                                    inputs do not). It was stored as +-65504,
                                    never as an infinity; the bit stays set
                                    until isvd_init. */

/* Config flags. */
#define ISKV_NO_COORD_SYNC 1 /* basis-only ablation (iS-KV notes §2.3): merges
                                replace the basis but never rewrite the stored
                                coordinates of old rows */
#define ISKV_NO_GRAPH 2      /* enqueue every kernel of a merge or
                                re-orthogonalisation directly. By default, on a
                                non-null stream, the fixed launch sequence is
                                recorded once into a HIP graph (per block size)
                                and replayed; results are the same. */
#define ISKV_FROZEN_BASIS 4  /* frozen-basis baseline (iS-KV notes §6.4 ablation,
                                §8): merges keep B and every stored row as they
                                are and append only the new rows' coordinates
                                F B; no residual, core solve, coordinate rewrite,
                                basis update or re-orthogonalisation */
#define ISKV_BF16_COORDS 8   /* persistent 2-byte factors (iS-KV notes §4.4, §7.3):
                                the coordinates C are stored as bf16 ([n_cap x
                                r_max] uint16, round to nearest even), every
                                product still computed in fp32; B and sigma
                                stay fp32. The rounding of the stored rows at
                                each merge is the factor drift of eq.(14). */
#define ISKV_FP16_COORDS 16  /* persistent fp16 factors (iS-KV notes §7.3): C is
                                stored as IEEE half ([n_cap x r_max] uint16 bits,
                                round to nearest even), products in fp32 as
                                above. Overflow guard: a value above 65504 in
                                magnitude is stored as +-65504 (saturated) and
                                latches ISKV_DEV_FP16_OVERFLOW. Exclusive with
                                ISKV_BF16_COORDS. */

/* Output dtypes of kv_reconstruct. */
#define ISKV_OUT_BF16 0
#define ISKV_OUT_FP32 1

/* ---- iSVD handle --------------------------------------------------------- */
typedef struct iskv_config {
  int32_t D;                 /* feature width H_kv * d_h (iS-KV notes §2.1), a multiple
                                of 64 in 64..8192                                         */
  int32_t r_max;             /* rank budget r, 1..1024, r <= D                            */
  int32_t b_max;             /* largest pending block b, 1..64                            */
  int32_t n_cap;             /* row capacity of the compressed history                    */
  int32_t reorth_every_rows; /* re-orthogonalise whenever the folded-row counter crosses
                                a multiple of this (notes §4.4: 256); 0 = only on request */
  float resid_rel_tol;       /* delta of the residual threshold (notes §4.1), default 0:
                                keep residual direction j when
                                rho_j > max(delta*s, max(D,b)*2^-23*s),
                                s = max(sigma_1, rho_1)                                   */
  int32_t flags;             /* ISKV_NO_COORD_SYNC | ISKV_NO_GRAPH | ISKV_FROZEN_BASIS |
                                ISKV_BF16_COORDS | ISKV_FP16_COORDS, or 0 (at most
                                one of NO_COORD_SYNC and FROZEN_BASIS, at most one
                                of BF16_COORDS and FP16_COORDS)                                          */
} iskv_config;

typedef struct isvd_handle isvd_handle;

/* Bytes of device workspace one handle needs for `cfg` (256-byte aligned
 * sub-buffers). Returns 0 if cfg is invalid. */
size_t isvd_workspace_bytes(const iskv_config* cfg);

/* Create a handle over caller-owned device buffers and reset the history to
 * empty (n = k = 0). iS-KV notes §2.2: the history is X^ = C B^T where
 * C = U diag(sigma) holds one row of coordinates per token.
 *   C         device fp32 [n_cap x r_max] (bf16 under ISKV_BF16_COORDS, fp16
 *             under ISKV_FP16_COORDS):
 *             coordinates; zero-filled here.
 *   sigma     device fp32 [r_max]: singular values, descending.
 *   B         device fp32 [D x r_max]: shared orthonormal basis, column j is
 *             basis vector j (row d holds feature d's k coefficients).
 *   pos       device int32 [n_cap]: original token position of each row.
 *   workspace device buffer of >= isvd_workspace_bytes(cfg) bytes, 256-aligned.
 *   stream    hipStream_t as void*; all later calls on the handle use it.
 * On success *out receives the handle. Errors: EINVAL, EWORKSPACE, EHIP. */
int isvd_init(isvd_handle** out, const iskv_config* cfg, float* C, float* sigma, float* B,
              int32_t* pos, void* workspace, size_t ws_bytes, void* stream);

/* Fold one pending exact block into the history: Algorithm 2 and §4.1-§4.2 of
 * the iS-KV notes. Projects F on B, takes the residual (subtracting its
 * component along B twice), finds the residual basis P by a rank-revealing
 * eigendecomposition of E E^T with the threshold above, forms the core
 * Z = [[diag(sigma), 0], [F B, F P]] of eq.(7), takes its truncated SVD
 * (keeping r' = min(r_max, k + p)), rewrites every old row's coordinates
 * C <- C H[:k] (skipped under ISKV_NO_COORD_SYNC), appends the new rows
 * [F B, F P] H, and sets B <- [B, P] H, sigma <- sigma+. Re-orthogonalises
 * afterwards when the folded-row counter crosses a multiple of
 * reorth_every_rows.
 *   F      device fp32 [b x D], the b oldest pending exact rows.
 *   pos_F  device int32 [b], their original positions (copied into pos).
 *   b      1..b_max.
 * Errors: EINVAL (null pointer, b out of range), ECAPACITY (n + b > n_cap).
 * Non-finite input and a non-converged core are latched on the device
 * (ISKV_DEV_NONFINITE / ISKV_DEV_NOCONV, read by isvd_query), and so is a
 * saturated fp16 coordinate (ISKV_DEV_FP16_OVERFLOW). */
int isvd_merge_block(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t b);

/* One merge on each of `count` paths in a single launch sequence (the
 * data-parallel form of isvd_merge_block for many independent (sequence,
 * layer, K/V) paths, iS-KV notes §2.2 and Algorithm 2): block z is
 * F + z * F_stride (device fp32 [b x D]) with positions pos_F + z * pos_stride
 * (device int32 [b]); every kernel of the merge runs once over all paths.
 * Requirements: 1 <= count <= 4096; the handles are distinct, were created
 * with identical configurations and the same stream, and share one buffer
 * layout: each handle's C, sigma, B, pos and workspace lie at one common byte
 * offset from handle 0's (e.g. all carved from one allocation with a fixed
 * per-path stride). F_stride >= b * D, pos_stride >= b. Results equal `count`
 * separate isvd_merge_block calls; paths that cross the re-orthogonalisation
 * schedule together are re-orthogonalised in one batched sequence too.
 * Errors: EINVAL (requirements), ECAPACITY (n + b > n_cap for a path). */
int isvd_merge_block_batched(isvd_handle* const* hs, int32_t count, const float* F, int64_t F_stride,
                             const int32_t* pos_F, int64_t pos_stride, int32_t b);

/* Re-orthogonalise the factors: iS-KV notes §4.4. Equivalent to the notes'
 * thin QR of U and B and SVD of R_U diag(sigma) R_B^T: the product C B^T is
 * kept, B becomes orthonormal and C's columns orthogonal with norms sigma.
 * Errors: EMODE under ISKV_NO_COORD_SYNC (the stale rows have no consistent
 * factorisation to re-orthogonalise) or ISKV_FROZEN_BASIS (B is frozen). */
int isvd_reorth(isvd_handle* h);

/* Switch the merge mode of a handle between calls (the baselines the iS-KV
 * notes compare the full merge against): `mode` is 0 (full merge, §4),
 * ISKV_NO_COORD_SYNC (basis-only ablation, §2.3) or ISKV_FROZEN_BASIS (frozen
 * basis, §6.4 / §8); the handle's other flags are kept. Typical use: fold a
 * prompt with full merges, then freeze its basis. Leaving the frozen mode for
 * the full merge enqueues a re-orthogonalisation (§4.4) first, since the
 * appended coordinates F B are not orthogonal columns with norms sigma; no
 * other switch changes the factors. Recorded launch sequences are dropped and
 * recorded again on the next call.
 * Errors: EINVAL (null handle, another bit in mode, both bits), EHIP. */
int isvd_set_mode(isvd_handle* h, int32_t mode);

/* Synchronise the handle's stream and read the device counters: rows n,
 * current rank k and the device status word (ISKV_DEV_* bits). Any pointer
 * may be NULL. Errors: EHIP. */
int isvd_query(isvd_handle* h, int32_t* n, int32_t* k, int32_t* status);

/* Diagnostic: synchronise the stream and copy the first `count` (<= 16)
 * device state words of the handle: [0] n, [1] k, [2] p of the last merge,
 * [3] folded rows, [4] status bits, [5] core width k + p, [6] r',
 * [7] Jacobi sweeps of the last fallback solve, [11] core eigensolver flags
 * (1 converged by parallel refinement, 2 single-workgroup Jacobi fallback),
 * [12] refinement steps of the last core solve, [14] Jacobi sweeps of the last
 * residual eigensolve. Errors: EINVAL, EHIP. */
int isvd_query_state(isvd_handle* h, int32_t* state, int32_t count);

/* Run the handle's core eigensolver on a caller matrix (the step of
 * Algorithm 2 that takes the SVD of the core, iS-KV notes §4.2, exposed so it
 * can be checked on its own): A is device fp64 [m x m], symmetric,
 * row-major; on return lam (device fp64 [m]) holds its eigenvalues in
 * descending order and V (device fp64 [m x m], row-major) the matching
 * orthonormal eigenvectors as columns. m <= r_max + b_max. Uses the handle's
 * workspace and stream (do not interleave with a merge in flight); leaves
 * the factors untouched. Errors: EINVAL, EHIP. */
int isvd_sym_eig(isvd_handle* h, const double* A, int32_t m, double* lam, double* V);

/* Instrumentation: with on != 0, the handle's following merges run their
 * kernels one by one (no recorded launch sequence) with a HIP event at each
 * of the five stage boundaries of Algorithm 2 (iS-KV notes §4.1-§4.3);
 * on == 0 switches back. Creates the events on first use. Errors: EINVAL,
 * EHIP. */
int isvd_set_timing(isvd_handle* h, int32_t on);

/* Waits for the last timed merge and writes the durations of its stages in
 * milliseconds to ms[0..count-1] (entries past 5 get 0): [0] projection and
 * residual (Q = F B, E = F - Q B^T twice), [1] residual basis (E E^T, its
 * eigendecomposition, P, F P), [2] core Gram and its eigendecomposition,
 * [3] coordinate update of the old rows (C <- C H[:k]), [4] new rows, basis
 * update and bookkeeping. Errors: EINVAL, EMODE (timing off or no merge
 * timed since it was switched on), EHIP. */
int isvd_stage_times(isvd_handle* h, float* ms, int32_t count);

/* Rows folded so far (host-side, no sync). */
int32_t isvd_rows(const isvd_handle* h);

/* Copy one path's compressed history into another handle: C (rows 0..n-1),
 * sigma, B and its bf16 copy, the positions and the device state words (n, k,
 * the folded-row counter), i.e. the factor U diag(sigma) B^T of one
 * (sequence, layer, K/V) path of iS-KV notes §2.2 with its row positions
 * (Algorithm 3). The two paths are independent afterwards: this forks a
 * sequence whose continuations are compressed separately.
 *   dst, src  handles with the same D, r_max, b_max, coordinate storage and
 *             merge mode; dst's n_cap >= src's row count.
 * Enqueued on dst's stream as device-to-device copies; src's pending work on
 * another stream must be complete (the caller synchronises). dst's own
 * history is replaced. Errors: EINVAL (mismatched handles, dst == src),
 * ECAPACITY, EHIP. */
int isvd_copy(isvd_handle* dst, const isvd_handle* src);

/* Release the host handle (device buffers stay the caller's). NULL is a no-op. */
void isvd_destroy(isvd_handle* h);

/* ---- reconstruction ------------------------------------------------------ */
/* Rebuild the dense cache in original position order: Algorithm 3 and §3.2 /
 * §5 of the iS-KV notes. Row pos[i] of `out` gets the compressed row C_i B^T
 * (i < n); row pos_exact[e] gets X_exact[e]; with apply_rope every row t is
 * then turned per head at position t (pairs (j, j + head_dim/2) by angle
 * t * rope_theta^(-2j/head_dim)), which is how the notes restore pre-RoPE
 * keys. Exact slots with pos_exact[e] < 0 are skipped, so a window buffer
 * with empty slots can be passed as is.
 *   h           handle whose history is read (not modified).
 *   X_exact     device fp32 [n_exact x D] or NULL when n_exact == 0.
 *   pos_exact   device int32 [n_exact].
 *   n_total     rows of out; the compressed and valid exact positions must
 *               partition 0..n_total-1 (the caller's contract); a position
 *               outside 0..n_total-1 is dropped, never written.
 *   head_dim    d_h, even, dividing 128 when D % 128 == 0, else dividing 64.
 *   out         device [n_total x D], bf16 bits (ISKV_OUT_BF16) or fp32
 *               (ISKV_OUT_FP32). fp32 output computes the product in fp32.
 *               bf16 output rounds C and B to bf16 (round to nearest even)
 *               and accumulates in fp32 on the matrix cores when
 *               D % 128 == 0, head_dim is 32, 64 or 128 and r_max % 8 == 0;
 *               otherwise it computes in fp32 and rounds the result.
 *   stream      hipStream_t as void* (NULL = the handle's stream).
 * Errors: EINVAL. */
int kv_reconstruct(const isvd_handle* h, const float* X_exact, const int32_t* pos_exact,
                   int32_t n_exact, int32_t n_total, int32_t head_dim, int32_t apply_rope,
                   float rope_theta, void* out, int32_t out_dtype, void* stream);

/* The compressed rows of several histories rebuilt by one launch (Algorithm 3
 * and §3.2 / §5 of the iS-KV notes, as kv_reconstruct without exact rows):
 * for every path i, row pos_i[j] of outs[i] gets C_i[j] B_i^T (j < n_i),
 * turned per head at that position when apply_rope[i] (keys on, values off).
 * One launch serves all paths, so its fixed cost (the launch, each
 * workgroup's basis operands, the pipeline's fill and drain) is paid once;
 * the bytes of every path are the same as with kv_reconstruct, and each
 * output equals kv_reconstruct(hs[i], NULL, NULL, 0, n_totals[i], head_dim,
 * apply_rope[i], rope_theta, outs[i], ISKV_OUT_BF16, stream) bit for bit.
 * The exact rows of each path go through kv_scatter_exact afterwards.
 *   hs          host array of count handles (1 <= count <=
 *               ISKV_RECON_MAX_PATHS), sharing D, r_max and the coordinate
 *               storage (ISKV_BF16_COORDS / ISKV_FP16_COORDS); not modified.
 *   outs        host array of count device pointers, bf16 [n_totals[i] x D].
 *   n_totals    host array: rows of each output, at least that handle's n.
 *   apply_rope  host array of count flags.
 *   head_dim    32, 64 or 128 (dividing 128); D a multiple of 128; r_max a
 *               multiple of 32, at most 256, or at most 512 when D is a
 *               multiple of 256 (the streaming bf16 matrix-core kernel's
 *               shapes: any other shape is EINVAL, use kv_reconstruct).
 *   stream      hipStream_t as void* (NULL = hs[0]'s stream); the caller
 *               orders the call after every handle's pending merges.
 * Errors: EINVAL. */
#define ISKV_RECON_MAX_PATHS 32
int kv_reconstruct_batched(isvd_handle* const* hs, int32_t count, void* const* outs, const int32_t* n_totals,
                           const int32_t* apply_rope, int32_t head_dim, float rope_theta, void* stream);

/* The exact-row half of kv_reconstruct on its own (Algorithm 3 and §3.2 of
 * the iS-KV notes): row pos_exact[e] of `out` gets X_exact[e], turned per
 * head at that position when apply_rope (same convention as kv_reconstruct);
 * slots with a position outside 0..n_total-1 (e.g. empty window slots, -1)
 * are skipped. Together with kv_reconstruct(h, NULL, NULL, 0, ...) it writes
 * exactly what kv_reconstruct with the exact rows writes.
 *   X_exact device fp32 [n_exact x D]; pos_exact device int32 [n_exact];
 *   head_dim even and dividing D; out device [n_total x D] of out_dtype.
 * Errors: EINVAL. */
int kv_scatter_exact(const float* X_exact, const int32_t* pos_exact, int32_t n_exact, int32_t D,
                     int32_t n_total, int32_t head_dim, int32_t apply_rope, float rope_theta,
                     void* out, int32_t out_dtype, void* stream);

/* ---- attention ----------------------------------------------------------- */
/* Dense GQA decode attention over a reconstructed cache: Algorithm 3 and
 * §2.1 of the iS-KV notes. For every batch row and query head h,
 *   o_h = softmax_t(scale * q_h . K[t, g]) V[t, g],  g = h / (Hq / Hkv),
 * over all n cached positions (no causal mask at decode; queries already
 * rotated). fp32 accumulation, bf16 output.
 *   q    device bf16 [batch x Hq x dh];  K, V device bf16 [batch x n x Hkv x dh]
 *   out  device bf16 [batch x Hq x dh]
 *   workspace  >= decode_attend_workspace_bytes(batch, n, Hq, dh) bytes.
 * Limits: dh == 128, Hq % Hkv == 0, Hq / Hkv <= 16, n >= 1.
 * Errors: EINVAL, EWORKSPACE. */
size_t decode_attend_workspace_bytes(int32_t batch, int32_t n, int32_t Hq, int32_t dh);
int decode_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch,
                  int32_t n, int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out,
                  void* workspace, size_t ws_bytes, void* stream);

/* decode_attend for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels as decode_attend, with the partial
 * results in a fixed 8 MiB device array inside the library instead of a
 * caller workspace. Nothing is allocated, here or in the library.
 *   Limit: batch * Hq * ceil(n / 128) * 520 bytes <= 8 MiB (for example
 *   Hq = 32 with batch * n <= 64,512 rows); larger calls return
 *   ISKV_EWORKSPACE before anything is enqueued.
 *   stream must belong to the current device (EINVAL otherwise). The first
 *   call on a device looks up that device's copy of the array.
 *   Every call on one device shares its array: calls that may overlap on one
 *   device (concurrent streams, or host threads) race and must be
 *   serialised by the caller. Each call writes every partial it reads, so
 *   nothing carries over from the previous call.
 * Arguments, limits and other errors as decode_attend. */
int decode_attend_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch, int32_t n,
                          int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out, void* stream);

/* Decode attention with the value history kept factored (the value-side
 * decode the iS-KV notes point to in §5.2 and §6: attend with the factors
 * rather than rebuilding the dense value cache). One sequence. For query
 * head h on KV head g = h / (Hq / Hkv), with p_h the softmax over every
 * position t of scale * K[t, g] . q_h:
 *   out_h = (p_h[pos]^T C) B[g dh : (g + 1) dh, :k]^T + p_h[pos_exact]^T X_exact[:, g dh : (g + 1) dh]
 * where C (n x k), B and pos are the value handle hv's coordinates, basis and
 * row positions, so the value side reads n k coordinates instead of n D values.
 *   q          device bf16 [Hq x dh], already rotated.
 *   K          device bf16 [n_total x Hkv x dh]: the key cache in position order.
 *   hv         the value path (read only); D = Hkv dh, r_max % 4 == 0, r_max <= 448.
 *   X_exact    device fp32 [n_exact x D] exact value rows at pos_exact (device
 *              int32 [n_exact]; slots with a position outside 0..n_total-1 are
 *              skipped, so a window buffer can be passed whole). The compressed and
 *              valid exact positions must partition 0..n_total-1.
 *   dh == 128, Hq <= 32, Hq / Hkv in {1, 2, 4}.
 *   out        device bf16 [Hq x dh].
 *   workspace  >= decode_attend_fv_workspace_bytes(hv, n_exact, Hq) bytes (sized
 *              for hv's row capacity); it holds partial results and per-head
 *              counters, so calls that may overlap must not share one.
 * Errors: EINVAL, EWORKSPACE, EHIP. */
size_t decode_attend_fv_workspace_bytes(const isvd_handle* hv, int32_t n_exact, int32_t Hq);
int decode_attend_fv(const uint16_t* q, const uint16_t* K, const isvd_handle* hv, const float* X_exact,
                     const int32_t* pos_exact, int32_t n_exact, int32_t n_total, int32_t Hq, int32_t Hkv,
                     int32_t dh, float scale, uint16_t* out, void* workspace, size_t ws_bytes, void* stream);

/* ---- prompt initialisation ----------------------------------------------- */
/* Replace the history by a fresh rank-k truncated SVD of the rows X (iS-KV
 * notes Algorithm 1: the non-exact prompt rows; §3.2: the value first
 * refit over the rebuilt prompt values plus the first rows to leave the
 * window), k = min(r_max, n, D). The handle is reset to these n rows. With
 * iters > 0 the factor is the truncated SVD itself, reached through the
 * Gram G = X^T X in fp64: `iters` subspace iterations V <- orth(G V) on a
 * block of l = min(r_max + b_max, n, D) columns (CholeskyQR in fp64 of the
 * column-normalised G V), then the Rayleigh-Ritz step (the l x l matrix
 * V^T G V solved by the block Jacobi), B = the top k Ritz vectors, sigma the
 * Ritz singular values and C = X B. The subspace error shrinks by
 * sigma_{l+1}^2 / sigma_k^2 per iteration, which the b_max extra columns
 * keep below 1 however close sigma_k and sigma_{k+1} are: about 15
 * iterations reach the oracle's SVD to 1e-6 on the key stream
 * (exp(-i/40) + 0.01, r = 192, b = 64) and 40 to 1e-5 on the value stream
 * ((1+i)^-1/2, r = 320). iters = 0 folds the rows by merges instead
 * (Algorithm 2), the incremental factor the refit replaces.
 *   X     device fp32 [n x D], rows in the order of pos.
 *   pos   device int32 [n], their original positions.
 *   work  device buffer of >= isvd_refit_workspace_bytes(h) bytes (not read
 *         when iters = 0): about D^2 + 2 D l doubles.
 * C <- X B stages 16 rows of X in LDS, so iters > 0 needs D <= 1984; the
 * block l must be at most 1024.
 * Errors: EINVAL (also D > 1984 or l > 1024 with iters > 0; iters > 64),
 * ECAPACITY (n > n_cap), EMODE (basis-only or frozen mode), EWORKSPACE,
 * EHIP; ISKV_DEV_NOCONV in the status word if the Ritz solve did not
 * converge in its sweep budget. */
size_t isvd_refit_workspace_bytes(const isvd_handle* h);
int isvd_refit(isvd_handle* h, const float* X, const int32_t* pos, int32_t n, int32_t iters, void* work,
               size_t work_bytes);

/* The value first refit (iS-KV notes §3.2): once r_V value rows have left the
 * recent window, the value path is rebuilt from its reconstructed history
 * (C B^T in the handle's row order, positions kept) followed by those rows,
 * by isvd_refit over the stacked rows; block folds take over afterwards.
 *   F      device fp32 [count x D], the rows that left the window (count >= 0).
 *   pos_F  device int32 [count], their positions.
 *   work   device buffer of >= isvd_value_first_refit_workspace_bytes(h)
 *          bytes (holds the stacked rows: about n_cap x D x 4 bytes).
 * Errors: as isvd_refit; ECAPACITY when history + count > n_cap. */
size_t isvd_value_first_refit_workspace_bytes(const isvd_handle* h);
int isvd_value_first_refit(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t count, int32_t iters,
                           void* work, size_t work_bytes);

/* Split the prompt's rows by their flags (iS-KV notes Algorithm 1):
 * row p (position pos0 + p) is kept exact when flags[p] & mask, otherwise it
 * belongs to the rows the path's factor is built from; both lists keep
 * position order. For the keys mask = 1 (E_K = P_K), for the values
 * mask = 6 (E_V = P_V | W_V), with the flags of iskv_prompt_protect.
 *   X        device fp32 [L x D], 16-byte aligned, D a multiple of 4.
 *   X_keep, pos_keep   device [L x D] fp32 / [L] int32 (either may be NULL
 *            to drop the exact rows or their positions); X_rest, pos_rest
 *            likewise for the other rows.
 *   counts   device int32 [2]: the exact and the other row counts (L = 0:
 *            both zero; X, flags and workspace are then not read).
 *   workspace  >= iskv_prompt_split_workspace_bytes(L) bytes.
 * Errors: EINVAL, EWORKSPACE, EHIP. */
size_t iskv_prompt_split_workspace_bytes(int32_t L);
int iskv_prompt_split(const float* X, const uint8_t* flags, int32_t L, int32_t D, uint32_t mask, int32_t pos0,
                      float* X_keep, int32_t* pos_keep, float* X_rest, int32_t* pos_rest, int32_t* counts,
                      void* workspace, size_t ws_bytes, void* stream);


/* Exact-row sets of a prompt (iS-KV notes §3.1, Algorithm 1), from
 * its post-RoPE keys. The prompt is cut into blocks of `block` tokens; the last
 * `suffix_blocks` whole blocks and the partial tail are the local suffix. For
 * each KV head and every other block, the anomaly score is the minimum over the
 * block's tokens of the cosine between the token's key and the block's mean key
 * (fp32; a cosine with a zero vector counts as 1). Each head keeps its
 * `per_head` lowest-scoring blocks (equal scores: lower block index first; NaN
 * scores last); P_K = union of the kept blocks over heads plus the suffix;
 * P_V = every position within v_radius of P_K; W_V = the last v_window
 * positions (W_K is empty). The notes use block 8, per_head 128, suffix 4,
 * v_radius 32, v_window 128.
 *   K_rot      device bf16 [L x Hkv x dh], the prompt's post-RoPE keys.
 *   flags      device uint8 [L]: bit 0 P_K, bit 1 P_V, bit 2 W_V. The exact
 *              sets are E_K = P_K and E_V = P_V | W_V.
 *   scores     device fp32 [Hkv x nb] or NULL: the block scores, nb =
 *              max(L / block - suffix_blocks, 0) scored blocks per head.
 *   workspace  >= iskv_prompt_protect_workspace_bytes(L, Hkv, block, suffix_blocks).
 * 1 <= block <= 64, 1 <= dh <= 256, per_head, suffix_blocks, v_radius,
 * v_window >= 0. Errors: EINVAL, EWORKSPACE, EHIP. */
size_t iskv_prompt_protect_workspace_bytes(int32_t L, int32_t Hkv, int32_t block, int32_t suffix_blocks);
int iskv_prompt_protect(const uint16_t* K_rot, int32_t L, int32_t Hkv, int32_t dh, int32_t block,
                        int32_t per_head, int32_t suffix_blocks, int32_t v_radius, int32_t v_window,
                        uint8_t* flags, float* scores, void* workspace, size_t ws_bytes, void* stream);

/* ---- exact window and pending FIFO --------------------------------------- */
/* The cache policy of §3.2 and Algorithm 3 (iS-KV notes): every new row is
 * stored exactly in a recent window of `window` rows; an unprotected row
 * leaving the window joins the pending FIFO and stays exact; once `block`
 * rows are pending they are folded by isvd_merge_block. Protected rows
 * (§3.1) stay exact for good.
 * The exact rows live in one caller-owned device buffer laid out as
 * [protected (prot_cap) | window ring (window) | pending (block)] rows of D
 * fp32, with a matching int32 position array (-1 marks an empty slot), so
 * that the whole buffer can be handed to kv_reconstruct as X_exact. */
typedef struct iskv_window iskv_window;

/* Rows of the exact buffer: prot_cap + window + block. */
int32_t iskv_window_rows(int32_t prot_cap, int32_t window, int32_t block);

/* rows: device fp32 [iskv_window_rows() x D]; pos: device int32 [same].
 * block must equal the b used for merges and be <= the handle's b_max.
 * Clears the position array. Errors: EINVAL, EHIP. */
int iskv_window_init(iskv_window** out, isvd_handle* h, int32_t prot_cap, int32_t window,
                     int32_t block, float* rows, int32_t* pos, void* stream);

/* Store `count` protected rows (device fp32 [count x D]) at host positions
 * pos_host[0..count-1]. Errors: ECAPACITY past prot_cap, EINVAL. */
int iskv_window_protect(iskv_window* w, const float* rows, const int32_t* pos_host,
                        int32_t count);

/* Append `count` new exact rows (device fp32 [count x D]) at consecutive
 * positions pos0, pos0+1, ...; rows pushed out of the window become pending
 * and every full block is merged into the handle. *merges (may be NULL)
 * receives the number of merges this call enqueued. Errors: EINVAL, and any
 * error of isvd_merge_block. */
int iskv_window_append(iskv_window* w, const float* rows, int32_t pos0, int32_t count,
                       int32_t* merges);

/* The same append on `count` windows in lockstep (one per independent path,
 * iS-KV notes §2.2), with every kernel run once over all of them and every
 * full block merged by isvd_merge_block_batched. Window z receives the n rows
 * at rows + z * rows_stride (device fp32, rows_stride >= n * D floats) at
 * positions pos0 .. pos0 + n - 1. Requirements (count >= 2): the windows are
 * distinct, have equal (prot_cap, window, block, D), the same stream and the
 * same history of appends and protected rows; their handles form a valid
 * isvd_merge_block_batched set; and every buffer of path z (the handle's C,
 * sigma, B, pos and workspace and the window's rows and pos) lies z * S
 * bytes after path 0's, for one stride S > 0 (one allocation carved at a
 * fixed per-path stride). count == 1 is iskv_window_append. Errors: EINVAL
 * (requirements), ECAPACITY (a merge would exceed a handle's n_cap; checked
 * before anything is enqueued), EHIP. */
int iskv_window_append_batched(iskv_window* const* ws, int32_t count, const float* rows,
                               int64_t rows_stride, int32_t pos0, int32_t n, int32_t* merges);

/* The exact buffer for kv_reconstruct: its rows, positions and slot count. */
int iskv_window_exact(const iskv_window* w, const float** rows, const int32_t** pos,
                      int32_t* count);

void iskv_window_destroy(iskv_window* w);

/* ---- misc ---------------------------------------------------------------- */
const char* iskv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ISKV_H */
