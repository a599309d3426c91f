"""Literal CPU oracle of the iS-KV hot path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the GPU path never does.

Source: Zhongzhu Zhou, reading notes on "iS-KV: Online Low-Rank KV Cache
Compression via Block-Incremental SVD" ("iS-KV notes" below). Symbols follow
the notes: the compressed history of one (layer, K-or-V) path is
U diag(sigma) B^T with U (n x k) and B (D x k) having orthonormal columns,
k <= r; a pending exact block F (b x D) is folded in by Algorithm 2.

Readings where the notes are silent or their formulas were lost:
  * residual threshold: keep rho_j > tau with
    tau = max(delta * s, max(D, b) * eps * s), s = max(sigma_1, rho_1),
    eps = 2**-23 (machine epsilon of the FP32 compute precision, §4.4), delta
    defaults to 0; p is capped at min(b, D - k);
  * ties between equal singular values are broken by LAPACK's order;
  * RoPE pairs feature j with j + d_h/2 inside each head, angle
    pos * theta**(-2j/d_h), no frequency scaling;
  * attention applies no causal mask at decode; query head h reads KV head
    floor(h / (H_q / H_kv)); queries arrive already rotated.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "EPS_FP32",
    "Factor",
    "empty_factor",
    "merge",
    "reorth",
    "fold_frozen",
    "truncated_factor",
    "prefill_init",
    "value_first_refit",
    "anomaly_block_scores",
    "prompt_protect",
    "persist_coords_bf16",
    "persist_coords_fp16",
    "fp16_round",
    "FP16_MAX",
    "represented",
    "stored_rows",
    "fresh_truncated_svd",
    "rope",
    "bf16_round",
    "reconstruct",
    "attend",
    "attend_factor_v",
    "persistent_bytes",
    "breakeven_rows",
    "dense_kv_bytes",
    "factor_drift",
    "one_step_drift",
    "run_stream",
]

# Machine epsilon of FP32, the compute precision of the update (iS-KV notes §4.4).
EPS_FP32 = 2.0 ** -23


@dataclass
class Factor:
    """One compressed path: history rows approximated by U diag(sigma) B^T.

    iS-KV notes §2.2: U (n x k) holds one row of coordinates per token, B
    (D x k) is the shared dictionary, sigma the k singular values, k <= r.
    ``pos`` keeps each row's original token position (§3.2, Algorithm 3).
    ``folded`` counts regular folded rows for the re-orthogonalisation
    schedule (§4.4). ``C_stale`` is set only in the basis-only ablation
    (§2.3): the stored coordinates of old rows are then never rewritten.
    """

    U: np.ndarray
    sigma: np.ndarray
    B: np.ndarray
    pos: np.ndarray
    folded: int = 0
    C_stale: np.ndarray | None = None
    dtype: type = np.float64
    fp16_overflow: bool = False  # a stored fp16 coordinate was saturated (§7.3 guard)

    @property
    def n(self) -> int:
        return self.U.shape[0]

    @property
    def k(self) -> int:
        return self.sigma.shape[0]

    @property
    def D(self) -> int:
        return self.B.shape[0]


def empty_factor(D: int, dtype=np.float64, sync: bool = True) -> Factor:
    """An empty history (n = k = 0)."""
    return Factor(U=np.zeros((0, 0), dtype), sigma=np.zeros((0,), dtype),
                  B=np.zeros((D, 0), dtype), pos=np.zeros((0,), np.int64), folded=0,
                  C_stale=None if sync else np.zeros((0, 0), dtype), dtype=dtype)


def _svd(a):
    u, s, vt = np.linalg.svd(a, full_matrices=False)
    return u, s, vt


def merge(fac: Factor, F: np.ndarray, pos_F, r: int, delta: float = 0.0,
          diag: dict | None = None) -> Factor:
    """Fold one pending exact block F (b x D) into the history (Algorithm 2).

    iS-KV notes §4.1-§4.2 and Algorithm 2:
      * empty history: the rank-r truncated SVD of F;
      * project onto the old basis, Q = F B, residual E = F - Q B^T, and
        subtract E's leftover component along B once more;
      * reduced QR of E^T = P_E R_E, SVD R_E = W diag(rho) V_E^T, keep the
        residual directions above the threshold: P = P_E W[:, :p];
        no residual directions when E = 0 or k = D;
      * core Z = [[diag(sigma), 0], [F B, F P]] of size (k+b) x (k+p), eq.(7);
      * truncated SVD of the core, Z ~ G diag(sigma+) H^T, keep r' = min(r, k+p);
      * old rows U <- U G_top, new rows G_bot, B+ = [B, P] H.
    The basis-only ablation (§2.3, eq.(3)) keeps the old rows' stored
    coordinates instead of rewriting them.
    """
    dt = fac.dtype
    F = np.asarray(F).astype(dt)
    b, D = F.shape
    assert D == fac.D
    pos_F = np.asarray(pos_F, dtype=np.int64).reshape(b)
    k = fac.k
    sync = fac.C_stale is None

    if k == 0:
        # Empty history: the rank-r truncated SVD of F (Algorithm 2, first case).
        G, s, Vt = _svd(F)
        rp = min(r, s.shape[0])
        U_new = G[:, :rp]
        sig_new = s[:rp]
        B_new = Vt[:rp].T
        if diag is not None:
            diag.update(dict(p=None, empty=True, s_plus=s, r_prime=rp))
        C_stale = None if sync else (U_new * sig_new[None, :])
        return Factor(U=U_new.astype(dt), sigma=sig_new.astype(dt), B=B_new.astype(dt),
                      pos=pos_F.copy(), folded=fac.folded + b, C_stale=C_stale, dtype=dt,
                      fp16_overflow=fac.fp16_overflow)

    B = fac.B
    # Projection and residual, with the second subtraction of the leftover
    # component along B (§4.1).
    Q = F @ B
    E = F - Q @ B.T
    E = E - (E @ B) @ B.T

    normE = np.linalg.norm(E)
    if k >= D or normE == 0.0:
        p = 0
        P = np.zeros((D, 0), dt)
        rho = np.zeros((0,), dt)
        tau = 0.0
    else:
        PE, RE = np.linalg.qr(E.T, mode="reduced")          # E^T = P_E R_E
        W, rho, _VEt = _svd(RE)                              # R_E = W diag(rho) V_E^T
        s_scale = max(float(fac.sigma[0]) if k > 0 else 0.0, float(rho[0]))
        tau = max(delta * s_scale, max(D, b) * EPS_FP32 * s_scale)
        p = int(np.count_nonzero(rho > tau))
        p = min(p, b, D - k)
        P = PE @ W[:, :p]

    FP = F @ P
    Z = np.zeros((k + b, k + p), dt)
    Z[:k, :k] = np.diag(fac.sigma)
    Z[k:, :k] = Q
    Z[k:, k:] = FP

    G, s_plus, Ht = _svd(Z)
    # Sign convention (the notes leave it open): each singular pair whose index
    # is an old direction is oriented so that H[j, j] >= 0, i.e. the basis
    # moves continuously. The synced product does not depend on it; the
    # basis-only ablation does.
    for j in range(min(k, Ht.shape[0])):
        if Ht[j, j] < 0:
            Ht[j] = -Ht[j]
            G[:, j] = -G[:, j]
    rp = min(r, k + p)
    Hc = Ht[:rp].T                      # (k+p) x r'
    G_top = G[:k, :rp]
    G_bot = G[k:, :rp]
    sig_new = s_plus[:rp]

    U_new = np.vstack([fac.U @ G_top, G_bot])
    B_new = np.hstack([B, P]) @ Hc

    C_stale = None
    if not sync:
        # Basis-only ablation: old rows keep their stored coordinates, padded
        # with zero columns when the rank grows; new rows get G_bot diag(sigma+).
        old = fac.C_stale
        pad = np.zeros((old.shape[0], rp), dt)
        w = min(rp, old.shape[1])
        pad[:, :w] = old[:, :w]
        C_stale = np.vstack([pad, G_bot * sig_new[None, :]])

    if diag is not None:
        diag.update(dict(empty=False, Q=Q, E=E, P=P, rho=rho, tau=tau, p=p, Z=Z, G=G,
                         s_plus=s_plus, Hc=Hc, r_prime=rp, FP=FP))
    return Factor(U=U_new, sigma=sig_new, B=B_new,
                  pos=np.concatenate([fac.pos, pos_F]), folded=fac.folded + b,
                  C_stale=C_stale, dtype=dt, fp16_overflow=fac.fp16_overflow)


def reorth(fac: Factor) -> Factor:
    """Periodic re-orthogonalisation (iS-KV notes §4.4).

    Thin QR U = Q_U R_U and B = Q_B R_B, SVD of the small matrix
    R_U diag(sigma) R_B^T = W S V^T, then U <- Q_U W, sigma <- S, B <- Q_B V.
    The product U diag(sigma) B^T is unchanged in exact arithmetic.
    """
    if fac.k == 0:
        return fac
    QU, RU = np.linalg.qr(fac.U, mode="reduced")
    QB, RB = np.linalg.qr(fac.B, mode="reduced")
    M = RU @ np.diag(fac.sigma) @ RB.T
    W, S, Vt = _svd(M)
    return Factor(U=QU @ W, sigma=S, B=QB @ Vt.T, pos=fac.pos.copy(), folded=fac.folded,
                  C_stale=fac.C_stale, dtype=fac.dtype, fp16_overflow=fac.fp16_overflow)


def persist_coords_bf16(fac: Factor) -> Factor:
    """Persistent 2-byte factors (iS-KV notes §7.3, with fp32 compute): the
    stored coordinates C = U diag(sigma) are rounded to bfloat16 whenever they
    are written; sigma and B keep full precision. Returns the factor whose
    U diag(sigma) equals the rounded C (columns with sigma = 0 stay zero)."""
    if fac.k == 0 or fac.n == 0:
        return fac
    C = bf16_round(fac.U * fac.sigma[None, :])
    safe = np.where(fac.sigma > 0, fac.sigma, 1.0)
    U = np.where(fac.sigma[None, :] > 0, C / safe[None, :], 0.0)
    return Factor(U=U, sigma=fac.sigma.copy(), B=fac.B.copy(), pos=fac.pos.copy(), folded=fac.folded,
                  C_stale=fac.C_stale, dtype=fac.dtype)


def persist_coords_fp16(fac: Factor) -> Factor:
    """Persistent fp16 factors with the overflow guard (iS-KV notes §7.3: with
    FP16 factors some coordinates passed the largest finite half, 65504,
    became infinite and led to NaN logits; the scale of the derived factor
    carries the singular values, so finite inputs do not keep it finite).
    The stored C = U diag(sigma) is rounded to half whenever it is written;
    a magnitude above 65504 is stored as +-65504 and the returned factor's
    ``fp16_overflow`` is set (it stays set). sigma and B keep full precision."""
    if fac.k == 0 or fac.n == 0:
        return fac
    C, over = fp16_round(fac.U * fac.sigma[None, :])
    safe = np.where(fac.sigma > 0, fac.sigma, 1.0)
    U = np.where(fac.sigma[None, :] > 0, C / safe[None, :], 0.0)
    return Factor(U=U, sigma=fac.sigma.copy(), B=fac.B.copy(), pos=fac.pos.copy(), folded=fac.folded,
                  C_stale=fac.C_stale, dtype=fac.dtype, fp16_overflow=fac.fp16_overflow or over)


def anomaly_block_scores(K_rot: np.ndarray, Hkv: int, dh: int, block: int = 8, suffix_blocks: int = 4):
    """Anomaly score of each prompt block (iS-KV notes §3.1, Algorithm 1).

    The prompt's post-RoPE keys K_rot (L x Hkv*dh) are cut into blocks of
    `block` tokens; the last `suffix_blocks` whole blocks and the partial tail
    form the local suffix and are not scored. For KV head g and block j the
    score is the minimum over the block's tokens of the cosine similarity
    between the token's key and the mean key of the block. Reading: a cosine
    with a zero vector counts as 1 (no anomaly signal). Returns the scores
    (Hkv x nb, float64, nb = scored blocks) and the first suffix position.
    """
    K_rot = np.asarray(K_rot, dtype=np.float64)
    L = K_rot.shape[0]
    nfull = L // block
    nb = max(nfull - suffix_blocks, 0)
    scores = np.zeros((Hkv, nb))
    for g in range(Hkv):
        for j in range(nb):
            X = K_rot[j * block:(j + 1) * block, g * dh:(g + 1) * dh]
            mu = X.mean(axis=0)
            nm = np.linalg.norm(mu)
            cos = []
            for t in range(block):
                nt = np.linalg.norm(X[t])
                cos.append(1.0 if nt == 0.0 or nm == 0.0 else float(X[t] @ mu) / (nt * nm))
            scores[g, j] = min(cos)
    return scores, nb * block


def prompt_protect(K_rot: np.ndarray, Hkv: int, dh: int, block: int = 8, per_head: int = 128,
                   suffix_blocks: int = 4, v_radius: int = 32, v_window: int = 128, scores=None):
    """The exact-row sets of the prompt (iS-KV notes §3.1, Algorithm 1).

    Each KV head selects its `per_head` lowest-scoring blocks (all of them when
    there are fewer; equal scores: the lower block index first); the positions
    of the union of the selected blocks over heads, plus the local suffix, are
    P_K. P_V is every prompt position within `v_radius` of a P_K position; W_V
    the last min(v_window, L) positions (W_K is empty). ``scores`` may supply
    the block scores (for checking a selection made from them). Returns
    boolean masks (P_K, P_V, W_V) of length L; E_K = P_K, E_V = P_V | W_V.
    """
    L = np.asarray(K_rot).shape[0]
    if scores is None:
        scores, s0 = anomaly_block_scores(K_rot, Hkv, dh, block, suffix_blocks)
    else:
        scores = np.asarray(scores, dtype=np.float64)
        s0 = scores.shape[1] * block
    nb = scores.shape[1]
    pk = np.zeros(L, dtype=bool)
    pk[s0:] = True
    for g in range(Hkv):
        order = sorted(range(nb), key=lambda j: (scores[g, j], j))
        for j in order[:per_head]:
            pk[j * block:(j + 1) * block] = True
    pv = np.zeros(L, dtype=bool)
    for p in np.nonzero(pk)[0]:
        pv[max(0, p - v_radius):min(L, p + v_radius + 1)] = True
    wv = np.zeros(L, dtype=bool)
    wv[max(0, L - v_window):] = True
    return pk, pv, wv


def truncated_factor(X: np.ndarray, pos, r: int) -> Factor:
    """A path's factor from the fresh rank-r truncated SVD of its rows
    (iS-KV notes §2.2; Algorithm 1). Reading: k = the number of the
    first min(r, n, D) singular values that are not zero."""
    X = np.asarray(X, dtype=np.float64)
    n, D = X.shape
    if n == 0:
        return empty_factor(D)
    u, sv, vt = _svd(X)
    k = int(np.count_nonzero(sv[:min(r, sv.shape[0])] > 0.0))
    return Factor(U=u[:, :k].copy(), sigma=sv[:k].copy(), B=vt[:k].T.copy(),
                  pos=np.asarray(pos, dtype=np.int64).copy(), folded=0)


def prefill_init(K_pre: np.ndarray, K_rot: np.ndarray, V: np.ndarray, Hkv: int, dh: int, r_K: int, r_V: int,
                 block: int = 8, per_head: int = 128, suffix_blocks: int = 4, v_radius: int = 32,
                 v_window: int = 128):
    """Prompt initialisation (iS-KV notes §3.1, Algorithm 1).

    The exact sets come from the post-RoPE keys: E_K = P_K and
    E_V = P_V | W_V (W_K is empty). Each path keeps its exact rows as they are
    and replaces the rest by the fresh truncated SVD of those rows in position
    order (rank r_K for the pre-RoPE keys, r_V for the values), with their
    positions saved. Returns (factor_K, factor_V, E_K, E_V), E as boolean
    masks of length L. The pending queue starts empty and the value first
    refit is still to come (value_first_refit).
    """
    pk, pv, wv = prompt_protect(K_rot, Hkv, dh, block, per_head, suffix_blocks, v_radius, v_window)
    E_K, E_V = pk, pv | wv
    idx = np.arange(np.asarray(K_pre).shape[0])
    fac_K = truncated_factor(np.asarray(K_pre)[~E_K], idx[~E_K], r_K)
    fac_V = truncated_factor(np.asarray(V)[~E_V], idx[~E_V], r_V)
    return fac_K, fac_V, E_K, E_V


def value_first_refit(fac_V: Factor, rows: np.ndarray, pos_rows, r_V: int) -> Factor:
    """The value first refit (iS-KV notes §3.2): once r_V value rows have
    left the recent window, the value path is rebuilt as the fresh rank-r_V
    truncated SVD of its reconstructed history followed by those rows, and
    block folds take over afterwards."""
    X = np.concatenate([represented(fac_V), np.asarray(rows, dtype=np.float64)], axis=0)
    pos = np.concatenate([fac_V.pos, np.asarray(pos_rows, dtype=np.int64)])
    return truncated_factor(X, pos, r_V)


def fold_frozen(C: np.ndarray, B: np.ndarray, pos, F: np.ndarray, pos_F):
    """Frozen-basis fold, the baseline of the iS-KV notes' §6.4 ablation and
    §8: the basis B (D x k) and every stored row keep their values; the b new
    rows are stored with their coordinates in B, F B. C holds the stored
    coordinates (n x k). Returns the coordinates and positions after the fold.
    """
    C = np.asarray(C)
    F = np.asarray(F, dtype=np.float64)
    return np.vstack([C, F @ B]), np.concatenate([np.asarray(pos), np.asarray(pos_F)])


def represented(fac: Factor) -> np.ndarray:
    """The history the factors represent, U diag(sigma) B^T (n x D)."""
    return (fac.U * fac.sigma[None, :]) @ fac.B.T


def stored_rows(fac: Factor) -> np.ndarray:
    """Rows as stored: equal to ``represented`` unless coordinates are stale."""
    if fac.C_stale is None:
        return represented(fac)
    return fac.C_stale @ fac.B.T


def fresh_truncated_svd(X: np.ndarray, r: int):
    """Best rank-r approximation of X in the Frobenius norm (iS-KV notes §2.2).

    Returns (X_r, discarded singular values).
    """
    u, s, vt = _svd(np.asarray(X, dtype=np.float64))
    rr = min(r, s.shape[0])
    Xr = (u[:, :rr] * s[:rr]) @ vt[:rr]
    return Xr, s[rr:]


def rope(X: np.ndarray, pos, head_dim: int, theta: float) -> np.ndarray:
    """Rotate each head's pre-RoPE key at its own position (iS-KV notes §3.1, §5.2).

    Rows of X are concatenated heads (D = H_kv * head_dim). Inside a head,
    feature j < head_dim/2 pairs with j + head_dim/2 and the pair turns by
    pos * theta**(-2j/head_dim). Computed in float64.
    """
    X = np.asarray(X, dtype=np.float64)
    n, D = X.shape
    half = head_dim // 2
    pos = np.asarray(pos, dtype=np.float64).reshape(n)
    j = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * j / head_dim)
    ang = pos[:, None] * inv[None, :]            # n x half
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(X)
    for h in range(D // head_dim):
        a = X[:, h * head_dim:h * head_dim + half]
        bb = X[:, h * head_dim + half:(h + 1) * head_dim]
        out[:, h * head_dim:h * head_dim + half] = a * c - bb * s
        out[:, h * head_dim + half:(h + 1) * head_dim] = bb * c + a * s
    return out


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (via float32, round-to-nearest-even); returns float64 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# Largest finite IEEE half-precision value, (2 - 2^-10) * 2^15.
FP16_MAX = 65504.0


def fp16_round(x: np.ndarray):
    """Round to IEEE half precision (via float32, the compute precision, then
    round-to-nearest-even) with the overflow guard of the persistent fp16
    factors: a magnitude above FP16_MAX is stored as +-FP16_MAX instead of an
    infinity. NaN stays NaN. Returns (values as float64, whether any
    magnitude was above FP16_MAX)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    over = np.abs(f) > FP16_MAX  # NaN compares false
    h = np.where(over, np.copysign(np.float32(FP16_MAX), f), f).astype(np.float16)
    return h.astype(np.float64), bool(over.any())


def reconstruct(fac: Factor, X_exact, pos_exact, n_total: int, head_dim: int,
                apply_rope: bool, theta: float = 500000.0) -> np.ndarray:
    """Dense cache in original position order (iS-KV notes §3.2, §5, Algorithm 3).

    Compressed rows are rebuilt from the factors and scattered to their own
    original positions, exact rows are placed at theirs, and keys are rotated
    per token at that position. Every position 0 .. n_total-1 must be covered
    exactly once. Returns float64 (n_total x D).
    """
    D = fac.D
    out = np.full((n_total, D), np.nan)
    covered = np.zeros(n_total, dtype=np.int64)
    if fac.n > 0:
        rows = stored_rows(fac)
        out[fac.pos] = rows
        np.add.at(covered, fac.pos, 1)
    X_exact = np.asarray(X_exact, dtype=np.float64).reshape(-1, D)
    pos_exact = np.asarray(pos_exact, dtype=np.int64).reshape(-1)
    if pos_exact.size:
        out[pos_exact] = X_exact
        np.add.at(covered, pos_exact, 1)
    if not np.all(covered == 1):
        raise ValueError("compressed and exact positions must partition 0..n_total-1")
    if apply_rope:
        out = rope(out, np.arange(n_total), head_dim, theta)
    return out


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Dense GQA decode attention over the whole cache (iS-KV notes §2.1, Algorithm 3).

    q: (batch, H_q, d_h); K, V: (batch, n, H_kv, d_h). Query head h reads KV
    head floor(h / (H_q / H_kv)); softmax over every cached position, float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Bt, Hq, dh = q.shape
    Hkv = K.shape[2]
    grp = Hq // Hkv
    out = np.zeros((Bt, Hq, dh))
    for bi in range(Bt):
        for h in range(Hq):
            g = h // grp
            logits = (K[bi, :, g, :] @ q[bi, h]) * scale
            m = logits.max()
            w = np.exp(logits - m)
            out[bi, h] = (w @ V[bi, :, g, :]) / w.sum()
    return out


def attend_factor_v(q: np.ndarray, K: np.ndarray, fac: Factor, X_exact, pos_exact,
                    scale: float) -> np.ndarray:
    """Decode attention with the value history kept factored (the value-side
    decode the iS-KV notes point to in §5.2 / §6: attend with the factors
    instead of rebuilding the dense value cache).

    One sequence: q (H_q, d_h); K (n_total, H_kv, d_h) in position order; the
    value path's factor ``fac`` (compressed rows at fac.pos) and its exact
    rows X_exact (n_e, D) at pos_exact. For query head h on KV head g,
    p_h = softmax over every position t of scale * K[t, g] . q_h; then
      o_h = (p_h[fac.pos]^T U diag(sigma)) B[g d_h : (g + 1) d_h, :]^T
            + p_h[pos_exact]^T X_exact[:, g d_h : (g + 1) d_h].
    The compressed and exact positions must partition 0 .. n_total - 1.
    Float64; returns (H_q, d_h).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    n_total, Hkv, dh = K.shape
    Hq = q.shape[0]
    grp = Hq // Hkv
    pos_c = np.asarray(fac.pos, dtype=np.int64).reshape(-1)
    pos_e = np.asarray(pos_exact, dtype=np.int64).reshape(-1)
    X_exact = np.asarray(X_exact, dtype=np.float64).reshape(-1, fac.D)
    allpos = np.concatenate([pos_c, pos_e])
    covered = np.zeros(n_total, dtype=np.int64)
    if allpos.size and (allpos.min() < 0 or allpos.max() >= n_total):
        raise ValueError("a position lies outside 0..n_total-1")
    np.add.at(covered, allpos, 1)
    if not np.all(covered == 1):
        raise ValueError("compressed and exact positions must partition 0..n_total-1")
    # stored coordinates of the compressed rows (C = U diag(sigma), or the
    # stale coordinates of the basis-only ablation)
    C = (fac.C_stale if fac.C_stale is not None else fac.U * fac.sigma[None, :]) if fac.n > 0 else None
    out = np.zeros((Hq, dh))
    for h in range(Hq):
        g = h // grp
        logits = (K[:, g, :] @ q[h]) * scale
        w = np.exp(logits - logits.max())
        p = w / w.sum()
        o = p[pos_e] @ X_exact[:, g * dh:(g + 1) * dh] if pos_e.size else np.zeros(dh)
        if fac.n > 0:
            y = p[pos_c] @ C
            o = o + y @ fac.B[g * dh:(g + 1) * dh, :].T
        out[h] = o
    return out


def persistent_bytes(n_c: int, n_e: int, D: int, r: int, beta_f: int, beta_e: int) -> int:
    """Persistent bytes of one path in one layer, eq.(12) (iS-KV notes §5.1).

    beta_f (n_c r + D r + r) for U, the shared basis B and the singular values,
    plus beta_e n_e D for the exact rows.
    """
    return beta_f * (n_c * r + D * r + r) + beta_e * n_e * D


def breakeven_rows(D: int, r: int) -> int:
    """Smallest compressed row count that saves bytes over dense storage (§5.1).

    With equal scalar widths the exact rows cancel and the factored history
    n r + D r + r undercuts the dense n D once n > r (D + 1) / (D - r).
    """
    n = 0
    while not (n * D > n * r + D * r + r):
        n += 1
    return n


def dense_kv_bytes(tokens: int, layers: int, D: int, bytes_per: int) -> int:
    """Dense K and V cache bytes of a model: tokens x layers x 2 x D x bytes."""
    return tokens * layers * 2 * D * bytes_per


def factor_drift(X: np.ndarray, X_inc: np.ndarray, r: int) -> float:
    """Excess relative error over a fresh same-rank SVD, eq.(14) (iS-KV notes §7.3)."""
    X = np.asarray(X, dtype=np.float64)
    nx = np.linalg.norm(X)
    Xr, _ = fresh_truncated_svd(X, r)
    return np.linalg.norm(X - X_inc) / nx - np.linalg.norm(X - Xr) / nx


def one_step_drift(fac: Factor, F, pos_F, r: int, delta: float = 0.0):
    """History drift of one merge, with and without coordinate sync (§2.3, eq.(3)).

    The reference is the history represented before the merge. Synced old rows
    are U G_top diag(sigma+) B+^T; basis-only old rows keep the old coordinates
    U diag(sigma) (zero-padded) and read them in the new basis B+.
    Returns (drift_sync, drift_basis_only, merged factor).
    """
    before = represented(fac)
    d = {}
    new = merge(fac, F, pos_F, r, delta, diag=d)
    n_old = fac.n
    synced_old = represented(new)[:n_old]
    C_old = fac.U * fac.sigma[None, :]
    rp = new.k
    pad = np.zeros((n_old, rp))
    w = min(rp, C_old.shape[1])
    pad[:, :w] = C_old[:, :w]
    basis_only_old = pad @ new.B.T
    nb = np.linalg.norm(before)
    return (np.linalg.norm(synced_old - before) / nb,
            np.linalg.norm(basis_only_old - before) / nb, new)


def run_stream(X: np.ndarray, b: int, r: int, reorth_every_rows: int = 0, delta: float = 0.0,
               dtype=np.float64, sync: bool = True, pos0: int = 0, fac: Factor | None = None,
               callback=None, persist_bf16: bool = False, persist_fp16: bool = False) -> Factor:
    """Fold the rows of X block by block (b rows each), in order.

    Re-orthogonalises whenever the folded-row counter reaches a multiple of
    ``reorth_every_rows`` (iS-KV notes §4.4; 0 disables it). ``callback`` is
    called after every merge with (merge index, factor). ``persist_bf16``
    (``persist_fp16``) rounds the stored coordinates to bfloat16 (to half,
    with the overflow guard) after every merge and re-orthogonalisation
    (persistent 2-byte factors, §7.3).
    """
    if persist_bf16 and persist_fp16:
        raise ValueError("one 2-byte format at a time")
    persist = persist_coords_bf16 if persist_bf16 else (persist_coords_fp16 if persist_fp16 else None)
    X = np.asarray(X)
    n = X.shape[0]
    if fac is None:
        fac = empty_factor(X.shape[1], dtype=dtype, sync=sync)
    for t, s in enumerate(range(0, n, b)):
        F = X[s:s + b]
        pos_F = np.arange(pos0 + s, pos0 + s + F.shape[0])
        before = fac.folded
        fac = merge(fac, F, pos_F, r, delta)
        if persist is not None:
            fac = persist(fac)
        if reorth_every_rows and sync and (fac.folded // reorth_every_rows) > (before // reorth_every_rows):
            fac = reorth(fac)
            if persist is not None:
                fac = persist(fac)
        if callback is not None:
            callback(t, fac)
    return fac
