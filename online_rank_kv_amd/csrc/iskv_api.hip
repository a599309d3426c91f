// C ABI of the gfx950 iS-KV library: argument checks, workspace carving,
// host-side bookkeeping of the exact window / pending FIFO, and dispatch to
// the kernel launchers. See include/iskv.h for the contract of every call.
#include "iskv_internal.h"

#include <new>
#include <stdlib.h>
#include <string.h>

#include <vector>

namespace {

constexpr size_t kAlign = 256;
constexpr int kGramSplits = 17;  // 16 row chunks of C + 1 slice for B

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool cfg_ok(const iskv_config* c) {
  if (!c) return false;
  if (c->D < 64 || c->D > 8192 || (c->D % 64) != 0) return false;
  if (c->r_max < 1 || c->r_max > c->D) return false;
  if (c->b_max < 1 || c->b_max > 64) return false;
  if (c->r_max + c->b_max > 1024) return false;
  if (c->n_cap < 1) return false;
  if (c->reorth_every_rows < 0) return false;
  if (!(c->resid_rel_tol >= 0.f)) return false;
  if (c->flags & ~(ISKV_NO_COORD_SYNC | ISKV_NO_GRAPH | ISKV_FROZEN_BASIS | ISKV_BF16_COORDS | ISKV_FP16_COORDS))
    return false;
  if ((c->flags & ISKV_BF16_COORDS) && (c->flags & ISKV_FP16_COORDS)) return false;
  if ((c->flags & ISKV_NO_COORD_SYNC) && (c->flags & ISKV_FROZEN_BASIS)) return false;
  return true;
}

// Layout of the workspace; when base == nullptr only the size is computed.
size_t carve(const iskv_config* c, char* base, isvd_ws* w) {
  const size_t D = c->D, R = c->r_max, Bm = c->b_max, M = c->r_max + c->b_max;
  const size_t LM = iskv_core_ld((int)M);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return p;
  };
  isvd_ws tmp;
  isvd_ws& x = w ? *w : tmp;
  x.st = (int32_t*)take(ST_COUNT * sizeof(int32_t));
  x.Bbf = (uint16_t*)take(D * R * 2);
  x.Q = (float*)take(Bm * R * 4);
  x.E = (float*)take(Bm * D * 4);
  x.EB = (float*)take(Bm * R * 4);
  x.GE = (double*)take(Bm * Bm * 8);
  x.VE = (double*)take(Bm * Bm * 8);
  x.rho = (double*)take(Bm * 8);
  x.P = (float*)take(D * Bm * 4);
  x.FP = (float*)take(Bm * Bm * 4);
  x.A = (double*)take(LM * LM * 8);
  x.V = (double*)take(LM * LM * 8);
  x.S = (double*)take(LM * LM * 8);
  x.W0 = (double*)take(LM * LM * 8);
  x.W1 = (double*)take(LM * LM * 8);
  x.T = (double*)take(LM * LM * 8);
  x.Km = (double*)take(LM * LM * 8);
  x.Pa = (double*)take(LM * LM * 8);
  x.Pb = (double*)take(LM * LM * 8);
  x.MB = (double*)take(LM * LM * 8);
  x.Zb = (double*)take(LM * LM * 8);
  x.naux = (int)((LM / 16) * (LM / 16));
  x.aux = (double*)take((size_t)x.naux * 8);
  x.edges = (int32_t*)take((size_t)ISKV_PCJ_EMAX * 2 * 4);
  {
    const size_t G = M / 2 + 1;  // rotation groups have at least two members
    x.itab = (int32_t*)take((2 * M + G * (1 + ISKV_PCJ_CMAX)) * 4);
    x.rtab = (double*)take((M + G * ISKV_PCJ_CMAX * ISKV_PCJ_CMAX) * 8);
  }
  x.Dp = (double*)take((LM / 16) * LM * 8);
  x.lam = (double*)take(M * 8);
  x.rot_cap = 0;
  x.rot = nullptr;
  x.Hc = (float*)take(M * R * 4);
  x.T2 = (float*)take(R * R * 4);
  x.sig_new = (float*)take(M * 4);
  x.gram_splits = kGramSplits;
  x.GC = (double*)take((size_t)kGramSplits * R * R * 8);
  x.GB = (double*)take(R * R * 8);
  x.RB = (double*)take(R * R * 8);
  x.order = (int32_t*)take(M * 4);
  x.Fs = (float*)take(Bm * D * 4);
  x.posFs = (int32_t*)take(Bm * 4);
  x.btab = (int64_t*)take(ISKV_MAX_BATCH * 8);
  return off;
}

}  // namespace

extern "C" {

const char* iskv_strerror(int status) {
  switch (status) {
    case ISKV_OK: return "ok";
    case ISKV_EINVAL: return "invalid argument";
    case ISKV_ECAPACITY: return "capacity exceeded";
    case ISKV_EWORKSPACE: return "workspace too small or misaligned";
    case ISKV_EHIP: return "HIP runtime error";
    case ISKV_ENONFINITE: return "non-finite values met on the device";
    case ISKV_ENOCONV: return "core eigensolver did not converge";
    case ISKV_EMODE: return "operation not available in this mode";
    default: return "unknown status";
  }
}

size_t isvd_workspace_bytes(const iskv_config* cfg) {
  if (!cfg_ok(cfg)) return 0;
  return carve(cfg, nullptr, nullptr) + kAlign;
}

// Empty history: n = k = 0, zero factors, no positions (enqueued on the stream).
static int reset_history(isvd_handle* h) {
  const iskv_config& c = h->cfg;
  hipStream_t s = h->stream;
  const size_t R = c.r_max;
  h->n_host = 0;
  h->folded_host = 0;
  ISKV_HIP_CHECK(hipMemsetAsync(h->w.st, 0, ST_COUNT * sizeof(int32_t), s));
  ISKV_HIP_CHECK(hipMemsetAsync(h->C, 0, (size_t)c.n_cap * R * iskv_coord_bytes(c), s));
  ISKV_HIP_CHECK(hipMemsetAsync(h->sigma, 0, R * sizeof(float), s));
  ISKV_HIP_CHECK(hipMemsetAsync(h->B, 0, (size_t)c.D * R * sizeof(float), s));
  ISKV_HIP_CHECK(hipMemsetAsync(h->w.Bbf, 0, (size_t)c.D * R * 2, s));
  ISKV_HIP_CHECK(hipMemsetAsync(h->pos, 0xff, (size_t)c.n_cap * sizeof(int32_t), s));
  return ISKV_OK;
}

int isvd_init(isvd_handle** out, const iskv_config* cfg, float* C, float* sigma, float* B,
              int32_t* pos, void* workspace, size_t ws_bytes, void* stream) {
  if (!out || !cfg_ok(cfg) || !C || !sigma || !B || !pos || !workspace) return ISKV_EINVAL;
  if (((uintptr_t)workspace) % kAlign != 0) return ISKV_EWORKSPACE;
  if (ws_bytes < carve(cfg, nullptr, nullptr)) return ISKV_EWORKSPACE;
  if (iskv_kernel_setup() != ISKV_OK) return ISKV_EHIP;
  isvd_handle* h = new (std::nothrow) isvd_handle();
  if (!h) return ISKV_EINVAL;
  h->cfg = *cfg;
  h->C = C; h->sigma = sigma; h->B = B; h->pos = pos;
  h->ws_base = workspace; h->ws_bytes = ws_bytes;
  h->stream = (hipStream_t)stream;
  h->m_max = cfg->r_max + cfg->b_max;
  h->ldm = iskv_core_ld(h->m_max);
  carve(cfg, (char*)workspace, &h->w);
  if (reset_history(h) != ISKV_OK) {
    delete h;
    return ISKV_EHIP;
  }
  *out = h;
  return ISKV_OK;
}

size_t isvd_refit_workspace_bytes(const isvd_handle* h) { return h ? iskv_refit_ws_bytes(h) : 0; }

int isvd_refit(isvd_handle* h, const float* X, const int32_t* pos, int32_t n, int32_t iters, void* work,
               size_t work_bytes) {
  if (!h || !X || !pos || n < 1 || iters < 0 || iters > 64) return ISKV_EINVAL;
  if (n > h->cfg.n_cap) return ISKV_ECAPACITY;
  if (h->cfg.flags & (ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS)) return ISKV_EMODE;
  if (iters > 0 && (!iskv_refit_supported(h->cfg) || iskv_refit_block(h) > 1024)) return ISKV_EINVAL;
  if (iters > 0 && (!work || work_bytes < iskv_refit_ws_bytes(h))) return ISKV_EWORKSPACE;
  int rc = reset_history(h);
  if (rc) return rc;
  if (iters == 0) {  // the incremental fold alone (Algorithm 2)
    for (int32_t s0 = 0; s0 < n; s0 += h->cfg.b_max) {
      const int32_t b = n - s0 < h->cfg.b_max ? n - s0 : h->cfg.b_max;
      rc = isvd_merge_block(h, X + (size_t)s0 * h->cfg.D, pos + s0, b);
      if (rc) return rc;
    }
    return ISKV_OK;
  }
  // the fp64 Gram, `iters` subspace iterations on an oversampled block, the
  // Rayleigh-Ritz step and C = X B (refit_gram.hip)
  ISKV_HIP_CHECK(hipMemcpyAsync(h->pos, pos, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToDevice, h->stream));
  h->n_host = n;
  h->folded_host = 0;
  return iskv_launch_refit_gram(h, X, n, iters, work);
}

// Workspace of the value first refit: the refit's, then B^T (r_max x D), the
// stacked rows (n_cap x D) and their positions (n_cap), 256-byte aligned.
static size_t vfr_offsets(const isvd_handle* h, size_t* o_bt, size_t* o_x, size_t* o_pos) {
  const iskv_config& c = h->cfg;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  *o_bt = al(iskv_refit_ws_bytes(h));
  *o_x = *o_bt + al((size_t)c.r_max * c.D * sizeof(float));
  *o_pos = *o_x + al((size_t)c.n_cap * c.D * sizeof(float));
  return *o_pos + al((size_t)c.n_cap * sizeof(int32_t));
}

size_t isvd_value_first_refit_workspace_bytes(const isvd_handle* h) {
  if (!h) return 0;
  size_t a, b, c;
  return vfr_offsets(h, &a, &b, &c);
}

int isvd_value_first_refit(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t count, int32_t iters,
                           void* work, size_t work_bytes) {
  if (!h || count < 0 || (count > 0 && (!F || !pos_F)) || iters < 0 || iters > 64) return ISKV_EINVAL;
  if (h->cfg.flags & (ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS)) return ISKV_EMODE;
  const int64_t n = (int64_t)h->n_host + count;
  if (n > h->cfg.n_cap) return ISKV_ECAPACITY;
  if (n == 0) return ISKV_OK;
  if (iters > 0 && !iskv_refit_supported(h->cfg)) return ISKV_EINVAL;
  size_t o_bt, o_x, o_pos;
  const size_t need = vfr_offsets(h, &o_bt, &o_x, &o_pos);
  if (!work || work_bytes < need) return ISKV_EWORKSPACE;
  char* wb = (char*)work;
  float* Xs = (float*)(wb + o_x);
  int32_t* Ps = (int32_t*)(wb + o_pos);
  const size_t D = h->cfg.D;
  const int32_t n_old = h->n_host;
  hipStream_t s = h->stream;
  // [reconstructed history; F] with positions [history's; pos_F]
  int rc = iskv_launch_materialize(h, Xs, (float*)(wb + o_bt));
  if (rc) return rc;
  if (n_old > 0)
    ISKV_HIP_CHECK(hipMemcpyAsync(Ps, h->pos, (size_t)n_old * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  if (count > 0) {
    ISKV_HIP_CHECK(hipMemcpyAsync(Xs + (size_t)n_old * D, F, (size_t)count * D * sizeof(float),
                                  hipMemcpyDeviceToDevice, s));
    ISKV_HIP_CHECK(hipMemcpyAsync(Ps + n_old, pos_F, (size_t)count * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  }
  return isvd_refit(h, Xs, Ps, (int32_t)n, iters, work, work_bytes);
}

// ---- prompt split ------------------------------------------------------------
size_t iskv_prompt_split_workspace_bytes(int32_t L) { return iskv_prompt_split_ws_bytes(L); }

int iskv_prompt_split(const float* X, const uint8_t* flags, int32_t L, int32_t D, uint32_t mask, int32_t pos0,
                      float* X_keep, int32_t* pos_keep, float* X_rest, int32_t* pos_rest, int32_t* counts,
                      void* workspace, size_t ws_bytes, void* stream) {
  if (!counts || L < 0 || D < 4 || D % 4 != 0 || pos0 < 0) return ISKV_EINVAL;
  if ((int64_t)pos0 + L > INT32_MAX) return ISKV_EINVAL;
  if (L > 0 && (!X || !flags || !workspace)) return ISKV_EINVAL;
  if ((uintptr_t)X % 16 || (uintptr_t)X_keep % 16 || (uintptr_t)X_rest % 16) return ISKV_EINVAL;
  if (ws_bytes < iskv_prompt_split_ws_bytes(L)) return ISKV_EWORKSPACE;
  return iskv_launch_prompt_split(X, flags, L, D, mask, pos0, X_keep, pos_keep, X_rest, pos_rest, counts, workspace,
                                  (hipStream_t)stream);
}

int32_t isvd_rows(const isvd_handle* h) { return h ? h->n_host : 0; }

int isvd_query_state(isvd_handle* h, int32_t* state, int32_t count) {
  if (!h || !state || count < 1 || count > ST_COUNT) return ISKV_EINVAL;
  int32_t st[ST_COUNT];
  ISKV_HIP_CHECK(hipStreamSynchronize(h->stream));
  ISKV_HIP_CHECK(hipMemcpy(st, h->w.st, sizeof(st), hipMemcpyDeviceToHost));
  for (int i = 0; i < count; ++i) state[i] = st[i];
  return ISKV_OK;
}

int isvd_merge_block(isvd_handle* h, const float* F, const int32_t* pos_F, int32_t b) {
  if (!h || !F || !pos_F) return ISKV_EINVAL;
  if (b < 1 || b > h->cfg.b_max) return ISKV_EINVAL;
  if ((int64_t)h->n_host + b > h->cfg.n_cap) return ISKV_ECAPACITY;
  int rc = iskv_launch_merge(h, F, pos_F, b);
  if (rc) return rc;
  const int before = h->folded_host;
  h->n_host += b;
  h->folded_host += b;
  const int T = h->cfg.reorth_every_rows;
  if (T > 0 && !(h->cfg.flags & (ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS)) && (h->folded_host / T) > (before / T)) {
    rc = iskv_launch_reorth(h);
    if (rc) return rc;
  }
  return ISKV_OK;
}

int isvd_merge_block_batched(isvd_handle* const* hs, int32_t count, const float* F, int64_t F_stride,
                             const int32_t* pos_F, int64_t pos_stride, int32_t b) {
  if (!hs || count < 1 || count > ISKV_MAX_BATCH || !F || !pos_F) return ISKV_EINVAL;
  isvd_handle* h0 = hs[0];
  if (!h0 || b < 1 || b > h0->cfg.b_max) return ISKV_EINVAL;
  if (F_stride < (int64_t)b * h0->cfg.D || pos_stride < b) return ISKV_EINVAL;
  const char* w0 = (const char*)h0->ws_base;
  for (int z = 0; z < count; ++z) {
    const isvd_handle* h = hs[z];
    if (!h || memcmp(&h->cfg, &h0->cfg, sizeof(iskv_config)) != 0 || h->stream != h0->stream)
      return ISKV_EINVAL;
    for (int y = 0; y < z; ++y)
      if (hs[y] == h) return ISKV_EINVAL;  // each handle once
    // one buffer layout: every buffer at the workspace's offset from handle 0
    const ptrdiff_t d = (const char*)h->ws_base - w0;
    if ((const char*)h->C - (const char*)h0->C != d || (const char*)h->sigma - (const char*)h0->sigma != d ||
        (const char*)h->B - (const char*)h0->B != d || (const char*)h->pos - (const char*)h0->pos != d)
      return ISKV_EINVAL;
    if ((int64_t)h->n_host + b > h->cfg.n_cap) return ISKV_ECAPACITY;
  }
  int rc = iskv_launch_merge_batched(hs, count, F, F_stride, pos_F, pos_stride, b);
  if (rc) return rc;
  const int T = h0->cfg.reorth_every_rows;
  bool lockstep = true;
  std::vector<isvd_handle*> due;
  for (int z = 0; z < count; ++z) {
    isvd_handle* h = hs[z];
    const int before = h->folded_host;
    h->n_host += b;
    h->folded_host += b;
    if (h->folded_host != h0->folded_host) lockstep = false;
    if (T > 0 && !(h->cfg.flags & (ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS)) && (h->folded_host / T) > (before / T))
      due.push_back(h);
  }
  if (due.empty()) return ISKV_OK;
  if (lockstep && (int)due.size() == count) return iskv_launch_reorth_batched(hs, count);
  for (isvd_handle* h : due) {
    rc = iskv_launch_reorth(h);
    if (rc) return rc;
  }
  return ISKV_OK;
}

int isvd_reorth(isvd_handle* h) {
  if (!h) return ISKV_EINVAL;
  if (h->cfg.flags & (ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS)) return ISKV_EMODE;
  return iskv_launch_reorth(h);
}

int isvd_set_mode(isvd_handle* h, int32_t mode) {
  const int32_t modes = ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS;
  if (!h || (mode & ~modes) || mode == modes) return ISKV_EINVAL;
  const int32_t old = h->cfg.flags & modes;
  if (old == mode) return ISKV_OK;
  iskv_release_graphs(h);
  h->cfg.flags = (h->cfg.flags & ~modes) | mode;
  // the appended coordinates F B are not orthogonal columns with norms sigma:
  // the full merge's core (eq.(7)) needs them re-orthogonalised first
  if ((old & ISKV_FROZEN_BASIS) && mode == 0 && h->n_host > 0) return iskv_launch_reorth(h);
  return ISKV_OK;
}

int isvd_query(isvd_handle* h, int32_t* n, int32_t* k, int32_t* status) {
  if (!h) return ISKV_EINVAL;
  int32_t st[ST_COUNT];
  ISKV_HIP_CHECK(hipStreamSynchronize(h->stream));
  ISKV_HIP_CHECK(hipMemcpy(st, h->w.st, sizeof(st), hipMemcpyDeviceToHost));
  if (n) *n = st[ST_N];
  if (k) *k = st[ST_K];
  if (status) *status = st[ST_STATUS];
  return ISKV_OK;
}

int isvd_copy(isvd_handle* dst, const isvd_handle* src) {
  if (!dst || !src || dst == src) return ISKV_EINVAL;
  const iskv_config& a = dst->cfg;
  const iskv_config& b = src->cfg;
  const int32_t same = ISKV_BF16_COORDS | ISKV_FP16_COORDS | ISKV_NO_COORD_SYNC | ISKV_FROZEN_BASIS;
  if (a.D != b.D || a.r_max != b.r_max || a.b_max != b.b_max || (a.flags & same) != (b.flags & same))
    return ISKV_EINVAL;
  const int32_t n = src->n_host;
  if (n > a.n_cap) return ISKV_ECAPACITY;
  hipStream_t s = dst->stream;
  const size_t R = a.r_max, D = a.D, es = iskv_coord_bytes(a);
  if (n > 0) {
    ISKV_HIP_CHECK(hipMemcpyAsync(dst->C, src->C, (size_t)n * R * es, hipMemcpyDeviceToDevice, s));
    ISKV_HIP_CHECK(hipMemcpyAsync(dst->pos, src->pos, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  }
  ISKV_HIP_CHECK(hipMemcpyAsync(dst->sigma, src->sigma, R * sizeof(float), hipMemcpyDeviceToDevice, s));
  ISKV_HIP_CHECK(hipMemcpyAsync(dst->B, src->B, D * R * sizeof(float), hipMemcpyDeviceToDevice, s));
  ISKV_HIP_CHECK(hipMemcpyAsync(dst->w.Bbf, src->w.Bbf, D * R * 2, hipMemcpyDeviceToDevice, s));
  ISKV_HIP_CHECK(hipMemcpyAsync(dst->w.st, src->w.st, ST_COUNT * sizeof(int32_t), hipMemcpyDeviceToDevice, s));
  dst->n_host = n;
  dst->folded_host = src->folded_host;
  return ISKV_OK;
}

void isvd_destroy(isvd_handle* h) {
  if (!h) return;
  iskv_release_graphs(h);
  for (hipEvent_t& e : h->tev)
    if (e) (void)hipEventDestroy(e);
  delete h;
}

int isvd_set_timing(isvd_handle* h, int32_t on) {
  if (!h) return ISKV_EINVAL;
  if (on && !h->tev[0]) {
    for (hipEvent_t& e : h->tev) ISKV_HIP_CHECK(hipEventCreate(&e));
  }
  h->timing = on != 0;
  h->timed = false;
  return ISKV_OK;
}

int isvd_stage_times(isvd_handle* h, float* ms, int32_t count) {
  if (!h || !ms || count < 1) return ISKV_EINVAL;
  if (!h->timing || !h->timed) return ISKV_EMODE;
  ISKV_HIP_CHECK(hipEventSynchronize(h->tev[ISKV_STAGES]));
  for (int i = 0; i < count; ++i) {
    ms[i] = 0.0f;
    if (i < ISKV_STAGES) ISKV_HIP_CHECK(hipEventElapsedTime(&ms[i], h->tev[i], h->tev[i + 1]));
  }
  return ISKV_OK;
}

int isvd_sym_eig(isvd_handle* h, const double* A, int32_t m, double* lam, double* V) {
  if (!h || !A || !lam || !V) return ISKV_EINVAL;
  if (m < 1 || m > h->m_max) return ISKV_EINVAL;
  return iskv_launch_sym_eig(h, A, m, lam, V);
}

int kv_reconstruct(const isvd_handle* h, const float* X_exact, const int32_t* pos_exact,
                   int32_t n_exact, int32_t n_total, int32_t head_dim, int32_t apply_rope,
                   float rope_theta, void* out, int32_t out_dtype, void* stream) {
  if (!h || !out) return ISKV_EINVAL;
  if (n_exact < 0 || (n_exact > 0 && (!X_exact || !pos_exact))) return ISKV_EINVAL;
  if (n_total < h->n_host || n_total < 0) return ISKV_EINVAL;
  if (head_dim < 2 || (head_dim & 1) || h->cfg.D % head_dim != 0) return ISKV_EINVAL;
  {
    const int W = (h->cfg.D % 128 == 0 && 128 % head_dim == 0) ? 128 : 64;
    if (W % head_dim != 0) return ISKV_EINVAL;
  }
  if (out_dtype != ISKV_OUT_BF16 && out_dtype != ISKV_OUT_FP32) return ISKV_EINVAL;
  if (apply_rope && !(rope_theta > 1.f)) return ISKV_EINVAL;
  hipStream_t s = stream ? (hipStream_t)stream : h->stream;
  return iskv_launch_reconstruct(h, X_exact, pos_exact, n_exact, n_total, head_dim, apply_rope,
                                 rope_theta, out, out_dtype, s);
}

int kv_reconstruct_batched(isvd_handle* const* hs, int32_t count, void* const* outs, const int32_t* n_totals,
                           const int32_t* apply_rope, int32_t head_dim, float rope_theta, void* stream) {
  if (!hs || !outs || !n_totals || !apply_rope) return ISKV_EINVAL;
  if (count < 1 || count > ISKV_RECON_MAX_PATHS) return ISKV_EINVAL;
  const uint32_t smask = ISKV_BF16_COORDS | ISKV_FP16_COORDS;
  for (int i = 0; i < count; ++i) {
    const isvd_handle* h = hs[i];
    if (!h || !outs[i]) return ISKV_EINVAL;
    if (h->cfg.D != hs[0]->cfg.D || h->cfg.r_max != hs[0]->cfg.r_max ||
        (h->cfg.flags & smask) != (hs[0]->cfg.flags & smask))
      return ISKV_EINVAL;
    if (n_totals[i] < h->n_host || n_totals[i] < 0) return ISKV_EINVAL;
    if (apply_rope[i] && !(rope_theta > 1.f)) return ISKV_EINVAL;
    if (!iskv_recon_stream_ok(h, n_totals[i], head_dim)) return ISKV_EINVAL;
  }
  hipStream_t s = stream ? (hipStream_t)stream : hs[0]->stream;
  return iskv_launch_reconstruct_batched(hs, count, (uint16_t* const*)outs, n_totals, apply_rope, head_dim,
                                         rope_theta, s, nullptr, nullptr, 0);
}

int kv_scatter_exact(const float* X_exact, const int32_t* pos_exact, int32_t n_exact, int32_t D,
                     int32_t n_total, int32_t head_dim, int32_t apply_rope, float rope_theta,
                     void* out, int32_t out_dtype, void* stream) {
  if (!out || n_exact < 0 || (n_exact > 0 && (!X_exact || !pos_exact))) return ISKV_EINVAL;
  if (D < 2 || n_total < 0) return ISKV_EINVAL;
  if (head_dim < 2 || (head_dim & 1) || D % head_dim != 0) return ISKV_EINVAL;
  if (out_dtype != ISKV_OUT_BF16 && out_dtype != ISKV_OUT_FP32) return ISKV_EINVAL;
  if (apply_rope && !(rope_theta > 1.f)) return ISKV_EINVAL;
  return iskv_launch_exact_rows(X_exact, pos_exact, n_exact, D, n_total, head_dim, apply_rope,
                                rope_theta, out, out_dtype, (hipStream_t)stream);
}

size_t decode_attend_workspace_bytes(int32_t batch, int32_t n, int32_t Hq, int32_t dh) {
  if (batch < 1 || n < 1 || Hq < 1 || dh != 128) return 0;
  return iskv_attend_ws_bytes(batch, n, Hq, dh);
}

int decode_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch,
                  int32_t n, int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !out || !workspace) return ISKV_EINVAL;
  if (batch < 1 || n < 1 || Hq < 1 || Hkv < 1 || dh != 128) return ISKV_EINVAL;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return ISKV_EINVAL;
  if (ws_bytes < decode_attend_workspace_bytes(batch, n, Hq, dh)) return ISKV_EWORKSPACE;
  return iskv_launch_attend(q, K, V, batch, n, Hq, Hkv, dh, scale, out, workspace, ws_bytes,
                            (hipStream_t)stream);
}

int decode_attend_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch, int32_t n,
                          int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out, void* stream) {
  if (!q || !K || !V || !out) return ISKV_EINVAL;
  if (batch < 1 || n < 1 || Hq < 1 || Hkv < 1 || dh != 128) return ISKV_EINVAL;
  if (Hq % Hkv != 0 || Hq / Hkv > 16) return ISKV_EINVAL;
  return iskv_launch_attend_noalloc(q, K, V, batch, n, Hq, Hkv, dh, scale, out, (hipStream_t)stream);
}

size_t decode_attend_fv_workspace_bytes(const isvd_handle* hv, int32_t n_exact, int32_t Hq) {
  if (!hv || n_exact < 0 || Hq < 1) return 0;
  return iskv_attend_fv_ws_bytes(hv->cfg.n_cap, n_exact, Hq, hv->cfg.r_max);
}

int decode_attend_fv(const uint16_t* q, const uint16_t* K, const isvd_handle* hv, const float* X_exact,
                     const int32_t* pos_exact, int32_t n_exact, int32_t n_total, int32_t Hq, int32_t Hkv,
                     int32_t dh, float scale, uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
  if (!q || !K || !hv || !out || !workspace) return ISKV_EINVAL;
  if (n_exact < 0 || (n_exact > 0 && (!X_exact || !pos_exact))) return ISKV_EINVAL;
  if (n_total < 1 || Hq < 1 || Hkv < 1 || dh != 128 || Hq > 32 || Hq % Hkv != 0) return ISKV_EINVAL;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4) return ISKV_EINVAL;
  if (hv->cfg.D != Hkv * 128 || hv->cfg.D > 1024) return ISKV_EINVAL;
  if (hv->cfg.r_max % 4 != 0 || hv->cfg.r_max > 448) return ISKV_EINVAL;  // a chunk of rows fits in LDS
  if (iskv_coord_bytes(hv->cfg) == 2 && hv->cfg.r_max % 8 != 0) return ISKV_EINVAL;  // 16-byte aligned 2-byte rows
  if (hv->n_host + n_exact < 1) return ISKV_EINVAL;
  if (ws_bytes < iskv_attend_fv_ws_bytes(hv->n_host, n_exact, Hq, hv->cfg.r_max)) return ISKV_EWORKSPACE;
  return iskv_launch_attend_fv(q, K, hv, X_exact, pos_exact, n_exact, n_total, Hq, Hkv, scale, out, workspace,
                               ws_bytes, (hipStream_t)stream);
}

// ---- prompt initialisation ---------------------------------------------------
size_t iskv_prompt_protect_workspace_bytes(int32_t L, int32_t Hkv, int32_t block, int32_t suffix_blocks) {
  return iskv_prompt_protect_ws_bytes(L, Hkv, block, suffix_blocks);
}

int iskv_prompt_protect(const uint16_t* K_rot, int32_t L, int32_t Hkv, int32_t dh, int32_t block,
                        int32_t per_head, int32_t suffix_blocks, int32_t v_radius, int32_t v_window,
                        uint8_t* flags, float* scores, void* workspace, size_t ws_bytes, void* stream) {
  if (!K_rot || !flags || !workspace) return ISKV_EINVAL;
  if (L < 1 || Hkv < 1 || dh < 1 || dh > 256 || block < 1 || block > 64) return ISKV_EINVAL;
  if (per_head < 0 || suffix_blocks < 0 || v_radius < 0 || v_window < 0) return ISKV_EINVAL;
  if ((int64_t)L * Hkv * dh > ((int64_t)1 << 31)) return ISKV_EINVAL;
  return iskv_launch_prompt_protect(K_rot, L, Hkv, dh, block, per_head, suffix_blocks, v_radius, v_window, flags,
                                    scores, workspace, ws_bytes, (hipStream_t)stream);
}

// ---- exact window and pending FIFO ----------------------------------------
int32_t iskv_window_rows(int32_t prot_cap, int32_t window, int32_t block) {
  if (prot_cap < 0 || window < 0 || block < 1) return 0;
  return prot_cap + window + block;
}

int iskv_window_init(iskv_window** out, isvd_handle* h, int32_t prot_cap, int32_t window,
                     int32_t block, float* rows, int32_t* pos, void* stream) {
  if (!out || !h || !rows || !pos) return ISKV_EINVAL;
  if (prot_cap < 0 || window < 0 || block < 1 || block > h->cfg.b_max) return ISKV_EINVAL;
  iskv_window* w = new (std::nothrow) iskv_window();
  if (!w) return ISKV_EINVAL;
  w->h = h;
  w->D = h->cfg.D;
  w->prot_cap = prot_cap;
  w->window = window;
  w->block = block;
  w->rows = rows;
  w->pos = pos;
  w->stream = (hipStream_t)stream;
  w->n_prot = 0;
  w->appended = 0;
  w->pending = 0;
  int total = prot_cap + window + block;
  if (iskv_launch_fill_pos(pos, total, -1, 0, w->stream) != ISKV_OK) {
    delete w;
    return ISKV_EHIP;
  }
  *out = w;
  return ISKV_OK;
}

int iskv_window_protect(iskv_window* w, const float* rows, const int32_t* pos_host, int32_t count) {
  if (!w || count < 0 || (count > 0 && (!rows || !pos_host))) return ISKV_EINVAL;
  if (w->n_prot + count > w->prot_cap) return ISKV_ECAPACITY;
  if (count == 0) return ISKV_OK;
  float* dst = w->rows + (size_t)w->n_prot * w->D;
  int rc = iskv_launch_window_move(dst, nullptr, rows, nullptr, 0, count, w->D, w->stream);
  if (rc) return rc;
  for (int i = 0; i < count; ++i) {
    rc = iskv_launch_fill_pos(w->pos + w->n_prot + i, 1, pos_host[i], 0, w->stream);
    if (rc) return rc;
  }
  w->n_prot += count;
  return ISKV_OK;
}

// Launch context of window moves: one window (bd = nullptr), or `bc` windows
// in lockstep whose buffers lie bd[z] bytes from window 0's, with the caller's
// rows of window z at src + z * src_stride floats.
struct win_batch {
  const int64_t* bd;
  int32_t bc;
  int64_t src_stride;
};

// Move `count` consecutive window slots starting at `slot` (wrapping) to dst.
static int move_from_ring(iskv_window* w, const win_batch& wb, int slot, int count, float* dst, int32_t* dpos) {
  const int D = w->D;
  float* win_rows = w->rows + (size_t)w->prot_cap * D;
  int32_t* win_pos = w->pos + w->prot_cap;
  int first = count < w->window - slot ? count : w->window - slot;
  int rc = iskv_launch_window_move(dst, dpos, win_rows + (size_t)slot * D, win_pos + slot, 0, first, D,
                                   w->stream, wb.bd, wb.bc, 1, 0);
  if (rc || first == count) return rc;
  return iskv_launch_window_move(dst + (size_t)first * D, dpos + first, win_rows, win_pos, 0,
                                 count - first, D, w->stream, wb.bd, wb.bc, 1, 0);
}

// Write `count` new rows (positions pos0..) into consecutive slots from `slot`.
static int write_to_ring(iskv_window* w, const win_batch& wb, int slot, const float* src, int32_t pos0,
                         int count) {
  const int D = w->D;
  float* win_rows = w->rows + (size_t)w->prot_cap * D;
  int32_t* win_pos = w->pos + w->prot_cap;
  int first = count < w->window - slot ? count : w->window - slot;
  int rc = iskv_launch_window_move(win_rows + (size_t)slot * D, win_pos + slot, src, nullptr, pos0,
                                   first, D, w->stream, wb.bd, wb.bc, 0, wb.src_stride);
  if (rc || first == count) return rc;
  return iskv_launch_window_move(win_rows, win_pos, src + (size_t)first * D, nullptr, pos0 + first,
                                 count - first, D, w->stream, wb.bd, wb.bc, 0, wb.src_stride);
}

// The append of Algorithm 1 (iS-KV notes §3.2): new rows enter the exact
// window, rows leaving it go to the pending FIFO, and every full pending block
// is merged. `ws` (count windows in lockstep, ws[0] == w) share w's counters;
// for count > 1 the kernels run batched and the merges go through
// isvd_merge_block_batched.
static int window_append(iskv_window* w, iskv_window* const* ws, int32_t count, isvd_handle* const* hs,
                         const win_batch& wb, const float* rows, int32_t pos0, int32_t n, int32_t* merges) {
  const int D = w->D;
  float* pend_rows = w->rows + (size_t)(w->prot_cap + w->window) * D;
  int32_t* pend_pos = w->pos + w->prot_cap + w->window;
  int done = 0;
  while (done < n) {
    // rows handled in this chunk: never more than fill the pending area once
    int c = n - done;
    if (c > w->block - w->pending) c = w->block - w->pending;
    const int64_t r = w->appended;
    int leave = 0;
    if (w->window > 0) {
      if (w->window < c) c = w->window;
      // rows r - window .. r - window + c - 1 leave the window (those that exist)
      int64_t first_out = r - w->window;
      int64_t lo = first_out < 0 ? 0 : first_out;
      int64_t hi = first_out + c;  // exclusive
      if (hi > lo) leave = (int)(hi - lo);
      if (leave > 0) {
        int rc = move_from_ring(w, wb, (int)(lo % w->window), leave, pend_rows + (size_t)w->pending * D,
                                pend_pos + w->pending);
        if (rc) return rc;
      }
      int rc = write_to_ring(w, wb, (int)(r % w->window), rows + (size_t)done * D, pos0 + done, c);
      if (rc) return rc;
    } else {
      int rc = iskv_launch_window_move(pend_rows + (size_t)w->pending * D, pend_pos + w->pending,
                                       rows + (size_t)done * D, nullptr, pos0 + done, c, D, w->stream, wb.bd,
                                       wb.bc, 0, wb.src_stride);
      if (rc) return rc;
      leave = c;
    }
    for (int z = 0; z < count; ++z) {
      ws[z]->pending += leave;
      ws[z]->appended += c;
    }
    done += c;
    if (w->pending == w->block) {
      int rc;
      if (count == 1) {
        rc = isvd_merge_block(w->h, pend_rows, pend_pos, w->block);
      } else {
        const int64_t fst = (const char*)hs[1]->ws_base - (const char*)hs[0]->ws_base;
        // every window's pending block lies at the common per-path byte stride
        rc = isvd_merge_block_batched(hs, count, pend_rows, fst / (int64_t)sizeof(float), pend_pos,
                                      fst / (int64_t)sizeof(int32_t), w->block);
      }
      if (rc) return rc;
      rc = iskv_launch_fill_pos(pend_pos, w->block, -1, 0, w->stream, wb.bd, wb.bc);
      if (rc) return rc;
      for (int z = 0; z < count; ++z) ws[z]->pending = 0;
      if (merges) (*merges)++;
    }
  }
  return ISKV_OK;
}

int iskv_window_append(iskv_window* w, const float* rows, int32_t pos0, int32_t count,
                       int32_t* merges) {
  if (merges) *merges = 0;
  if (!w || count < 0 || (count > 0 && !rows)) return ISKV_EINVAL;
  const win_batch wb = {nullptr, 1, 0};
  return window_append(w, &w, 1, &w->h, wb, rows, pos0, count, merges);
}

int iskv_window_append_batched(iskv_window* const* ws, int32_t count, const float* rows, int64_t rows_stride,
                               int32_t pos0, int32_t n, int32_t* merges) {
  if (merges) *merges = 0;
  if (!ws || count < 1 || count > ISKV_MAX_BATCH || n < 0 || (n > 0 && !rows)) return ISKV_EINVAL;
  iskv_window* w0 = ws[0];
  if (!w0) return ISKV_EINVAL;
  if (count == 1) return iskv_window_append(w0, rows, pos0, n, merges);
  if (rows_stride < (int64_t)n * w0->D) return ISKV_EINVAL;
  std::vector<isvd_handle*> hs(count);
  const char* r0 = (const char*)w0->rows;
  const char* p0 = (const char*)w0->pos;
  for (int z = 0; z < count; ++z)
    if (!ws[z] || !ws[z]->h) return ISKV_EINVAL;
  const char* b0 = (const char*)w0->h->ws_base;
  const ptrdiff_t d1 = (const char*)ws[1]->h->ws_base - b0;
  for (int z = 0; z < count; ++z) {
    const iskv_window* w = ws[z];
    if (w->D != w0->D || w->prot_cap != w0->prot_cap || w->window != w0->window ||
        w->block != w0->block || w->stream != w0->stream || w->h->stream != w0->stream ||
        w->n_prot != w0->n_prot || w->appended != w0->appended || w->pending != w0->pending)
      return ISKV_EINVAL;
    // window buffers at the same offsets as the handles' buffers, and one
    // stride from path to path (the pending blocks are passed to the batched
    // merge as F + z * stride)
    const ptrdiff_t d = (const char*)w->h->ws_base - b0;
    if ((const char*)w->rows - r0 != d || (const char*)w->pos - p0 != d) return ISKV_EINVAL;
    if (d1 <= 0 || d != (ptrdiff_t)z * d1 || d1 / (ptrdiff_t)sizeof(float) < (ptrdiff_t)w0->block * w0->D)
      return ISKV_EINVAL;
    for (int y = 0; y < z; ++y)
      if (ws[y] == w || ws[y]->h == w->h) return ISKV_EINVAL;
    hs[z] = w->h;
  }
  // capacity of every merge this call makes, checked before anything runs
  {
    int64_t app = w0->appended;
    int pend = w0->pending, nm = 0, done = 0;
    while (done < n) {
      int c = n - done;
      if (c > w0->block - pend) c = w0->block - pend;
      int leave = c;
      if (w0->window > 0) {
        if (w0->window < c) c = w0->window;
        int64_t first_out = app - w0->window, lo = first_out < 0 ? 0 : first_out, hi = first_out + c;
        leave = hi > lo ? (int)(hi - lo) : 0;
      }
      pend += leave;
      app += c;
      done += c;
      if (pend == w0->block) { ++nm; pend = 0; }
    }
    for (int z = 0; z < count; ++z)
      if ((int64_t)hs[z]->n_host + (int64_t)nm * w0->block > hs[z]->cfg.n_cap) return ISKV_ECAPACITY;
    if (nm > 0) {
      // the handles must also form a valid merge batch
      for (int z = 0; z < count; ++z)
        if (memcmp(&hs[z]->cfg, &hs[0]->cfg, sizeof(iskv_config)) != 0) return ISKV_EINVAL;
    }
  }
  int rc = iskv_upload_offsets(hs.data(), count);
  if (rc) return rc;
  const win_batch wb = {(const int64_t*)hs[0]->w.btab, count, rows_stride};
  return window_append(w0, ws, count, hs.data(), wb, rows, pos0, n, merges);
}

int iskv_window_exact(const iskv_window* w, const float** rows, const int32_t** pos, int32_t* count) {
  if (!w) return ISKV_EINVAL;
  if (rows) *rows = w->rows;
  if (pos) *pos = w->pos;
  if (count) *count = w->prot_cap + w->window + w->block;
  return ISKV_OK;
}

void iskv_window_destroy(iskv_window* w) { delete w; }

}  // extern "C"
