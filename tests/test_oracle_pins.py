"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, an invariant, a worked example the pages print (``tests/golden``), or a
textbook routine applied to a different matrix (brute force on tiny inputs).
None of them needs a GPU.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _orth(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def _factor_from(U, s, B, pos=None):
    n = U.shape[0]
    return O.Factor(U=U.copy(), sigma=np.asarray(s, float).copy(), B=B.copy(),
                    pos=np.arange(n) if pos is None else np.asarray(pos))


# ---------------------------------------------------------------- Eckart-Young
def test_eckart_young_known_spectrum():
    """Fresh truncated SVD error equals the root of the discarded sigma^2 (§2.2)."""
    rng = np.random.default_rng(1)
    n, d, r = 40, 12, 5
    s0 = np.array([9.0, 7.5, 5.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.25, 0.125, 0.0625])
    X = _orth(rng, n, d) @ np.diag(s0) @ _orth(rng, d, d).T
    Xr, disc = O.fresh_truncated_svd(X, r)
    expect = math.sqrt(float(np.sum(s0[r:] ** 2)))
    assert abs(np.linalg.norm(X - Xr) - expect) <= 1e-12 * np.linalg.norm(X)
    assert np.allclose(np.sort(disc)[::-1], s0[r:], rtol=1e-12, atol=1e-13)


def test_empty_history_merge_is_truncated_svd_of_block():
    """Empty history: the merge returns the rank-r SVD of F (Algorithm 2, first case)."""
    rng = np.random.default_rng(2)
    b, D, r = 8, 10, 3
    s0 = np.array([5.0, 4.0, 3.0, 2.0, 1.0, 0.5, 0.25, 0.1])
    F = _orth(rng, b, b) @ np.diag(s0) @ _orth(rng, D, b).T
    fac = O.merge(O.empty_factor(D), F, np.arange(b), r)
    assert fac.k == r and fac.n == b
    err = np.linalg.norm(O.represented(fac) - F)
    assert abs(err - math.sqrt(float(np.sum(s0[r:] ** 2)))) < 1e-12 * np.linalg.norm(F)
    assert np.allclose(fac.sigma, s0[:r], rtol=1e-12)


# ------------------------------------------------------- within the rank budget
def test_merge_within_budget_reproduces_stacked_matrix():
    """k + p <= r: the merge reproduces [U S B^T; F] exactly (§4.2, eq.(7))."""
    rng = np.random.default_rng(3)
    D, r = 16, 12
    U = _orth(rng, 9, 4)
    B = _orth(rng, D, 4)
    fac = _factor_from(U, [4.0, 3.0, 2.0, 1.0], B)
    target_old = O.represented(fac)
    F = rng.standard_normal((5, D))
    d = {}
    new = O.merge(fac, F, np.arange(9, 14), r, diag=d)
    assert d["p"] == 5 and new.k == 9
    stacked = np.vstack([target_old, F])
    assert np.linalg.norm(O.represented(new) - stacked) <= 1e-12 * np.linalg.norm(stacked)
    # orthonormal factors
    assert np.abs(new.U.T @ new.U - np.eye(new.k)).max() < 1e-12
    assert np.abs(new.B.T @ new.B - np.eye(new.k)).max() < 1e-12
    assert list(new.pos) == list(range(14))


def test_many_merges_exact_when_data_rank_fits():
    """A stream of rank-3 rows folded at r = 8 is reproduced exactly after every merge."""
    rng = np.random.default_rng(4)
    D = 20
    X = rng.standard_normal((64, 3)) @ rng.standard_normal((3, D))

    def cb(t, fac):
        seen = X[: fac.n]
        assert fac.k <= 8
        assert np.linalg.norm(O.represented(fac) - seen) <= 1e-11 * np.linalg.norm(seen)

    O.run_stream(X, 4, 8, callback=cb)


# ------------------------------------------------------------- pure rotation
def test_pure_rotation_merge_keeps_history_exact():
    """F inside span(B): no residual direction, synced history unchanged (§2.3, eq.(3))."""
    rng = np.random.default_rng(5)
    D, k = 12, 4
    U = _orth(rng, 10, k)
    B = _orth(rng, D, k)
    fac = _factor_from(U, [3.0, 2.5, 2.0, 1.5], B)
    F = rng.standard_normal((3, k)) @ B.T                     # F = A B^T
    ds, db, new = O.one_step_drift(fac, F, np.arange(10, 13), r=k)
    assert new.k == k
    stacked = np.vstack([O.represented(fac), F])
    assert np.linalg.norm(O.represented(new) - stacked) <= 1e-12 * np.linalg.norm(stacked)
    assert ds < 1e-13
    # the basis turned, so stale coordinates read in the new basis drift by O(1)
    assert db > 1e-2


def test_basis_only_drift_two_dim_closed_form():
    """2-D example (Fig. 3): a basis turned by theta moves stale rows by 2 sin(theta/2).

    History rows diag(2, 1) with B = I; one new row (1, 1); D = r = 2 so there
    is no residual. The core's right singular vectors are the eigenvectors of
    [[5, 1], [1, 2]], a rotation by theta with tan(2 theta) = 2/3.
    """
    fac = _factor_from(np.eye(2), [2.0, 1.0], np.eye(2))
    theta = 0.5 * math.atan2(2.0, 3.0)
    ds, db, new = O.one_step_drift(fac, np.array([[1.0, 1.0]]), [2], r=2)
    assert abs(db - 2.0 * math.sin(theta / 2.0)) < 1e-12
    assert ds < 1e-14
    assert abs(abs(new.B[0, 0]) - math.cos(theta)) < 1e-12
    # the same drift measured on the stored rows of a basis-only stream
    f2 = O.Factor(U=np.eye(2), sigma=np.array([2.0, 1.0]), B=np.eye(2), pos=np.arange(2),
                  C_stale=np.diag([2.0, 1.0]))
    m = O.merge(f2, np.array([[1.0, 1.0]]), [2], r=2)
    old = O.stored_rows(m)[:2]
    assert abs(np.linalg.norm(old - np.diag([2.0, 1.0])) / math.sqrt(5.0)
               - 2.0 * math.sin(theta / 2.0)) < 1e-12


# ------------------------------------------------------ local optimality, brute force
@pytest.mark.parametrize("seed", range(6))
def test_one_merge_is_best_rank_r_of_stacked_target(seed):
    """With the whole residual kept, one merge = best rank-r of [U S B^T; F] (§4.3)."""
    rng = np.random.default_rng(100 + seed)
    D, k, r, b = 7, 3, 4, 2
    fac = _factor_from(_orth(rng, 6, k), np.sort(rng.uniform(0.5, 3.0, k))[::-1], _orth(rng, D, k))
    F = rng.standard_normal((b, D))
    stacked = np.vstack([O.represented(fac), F])
    s_all = np.linalg.svd(stacked, compute_uv=False)
    if s_all[r - 1] - s_all[r] < 1e-6 * s_all[0]:
        pytest.skip("truncation tie: several best approximations")
    new = O.merge(fac, F, [6, 7], r)
    best, _ = O.fresh_truncated_svd(stacked, r)
    assert np.linalg.norm(O.represented(new) - best) <= 1e-11 * np.linalg.norm(stacked)
    # brute force: no other rank-r projection of the rows does better
    err_new = np.linalg.norm(O.represented(new) - stacked)
    for _ in range(50):
        V = _orth(rng, D, r)
        assert np.linalg.norm(stacked @ V @ V.T - stacked) >= err_new - 1e-12


def test_error_split_with_dropped_residual():
    """Dropped residual E_perp: error^2 = core tail + ||E_perp||^2 (§4.3)."""
    rng = np.random.default_rng(7)
    D, k, r, b = 10, 3, 4, 4
    fac = _factor_from(_orth(rng, 5, k), [4.0, 2.0, 1.0], _orth(rng, D, k))
    # residual singular values spread over decades so a threshold drops some
    base = fac.B @ rng.standard_normal((k, b))
    Pp = np.linalg.qr(np.hstack([fac.B, rng.standard_normal((D, b))]))[0][:, k:]
    F = (base + Pp @ np.diag([2.0, 0.5, 1e-3, 1e-4]) @ _orth(rng, b, b).T).T
    d = {}
    new = O.merge(fac, F, np.arange(5, 9), r, delta=1e-2, diag=d)
    assert d["p"] == 2
    stacked = np.vstack([O.represented(fac), F])
    E = d["E"]
    E_perp = E - E @ d["P"] @ d["P"].T
    lhs = np.linalg.norm(stacked - O.represented(new)) ** 2
    rhs = np.sum(d["s_plus"][r:] ** 2) + np.linalg.norm(E_perp) ** 2
    assert abs(lhs - rhs) <= 1e-10 * np.linalg.norm(stacked) ** 2
    # and E_perp carries exactly the two dropped residual singular values
    assert abs(np.linalg.norm(E_perp) ** 2 - (1e-3 ** 2 + 1e-4 ** 2)) < 1e-14


def test_residual_threshold_floor():
    """The scale-dependent floor keeps a real new direction and drops rounding-size ones (§4.1)."""
    rng = np.random.default_rng(8)
    D = 64
    B = _orth(rng, D, 4)
    fac = _factor_from(_orth(rng, 6, 4), [10.0, 8.0, 6.0, 4.0], B)
    Pp = np.linalg.qr(np.hstack([B, rng.standard_normal((D, 2))]))[0][:, 4:]
    tau = 64 * O.EPS_FP32 * 10.0
    for amp, expect_p in [(0.3 * tau, 0), (3.0 * tau, 1)]:
        F = (B @ rng.standard_normal(4) + amp * Pp[:, 0])[None, :]
        d = {}
        O.merge(fac, F, [6], r=8, diag=d)
        assert d["p"] == expect_p, (amp, d["rho"], d["tau"])


def test_full_rank_basis_adds_no_residual():
    """k = D: no residual direction is added, the merge still rotates (§4.2)."""
    rng = np.random.default_rng(9)
    D = 5
    fac = _factor_from(_orth(rng, 8, D), [5, 4, 3, 2, 1.0], _orth(rng, D, D))
    F = rng.standard_normal((2, D))
    d = {}
    new = O.merge(fac, F, [8, 9], r=D, diag=d)
    assert d["p"] == 0
    stacked = np.vstack([O.represented(fac), F])
    assert np.linalg.norm(O.represented(new) - stacked) <= 1e-12 * np.linalg.norm(stacked)


# ------------------------------------------------------------ worked example
def test_rank1_counterexample_matches_pages():
    """Path dependence (§4.3, Fig. 4): incremental sees 16 and 9, fresh best error 4."""
    g = json.load(open(os.path.join(GOLDEN, "rank1_counterexample.json")))
    r = g["rank_budget"]
    X1 = np.array(g["first_batch"])
    Fn = np.array(g["new_rows"])
    fac = O.merge(O.empty_factor(2), X1, [0, 1], r)
    d = {}
    new = O.merge(fac, Fn, [2], r, diag=d)
    assert np.allclose(np.sort(d["s_plus"] ** 2)[::-1], g["incremental_core_sigma_sq"], atol=1e-12)
    assert np.allclose(np.abs(new.B[:, 0]), g["incremental_keeps"], atol=1e-12)
    full = np.vstack([X1, Fn])
    best, disc = O.fresh_truncated_svd(full, r)
    assert abs(np.linalg.norm(full - best) - g["fresh_best_error"]) < 1e-12
    _, _, vt = np.linalg.svd(full)
    assert np.allclose(np.abs(vt[0]), g["fresh_keeps"], atol=1e-12)
    # incremental error against the whole history: the dropped e2 energy 9 + 9
    assert abs(np.linalg.norm(full - O.represented(new)) - math.sqrt(18.0)) < 1e-12


# --------------------------------------------------------------- reorth
def test_reorth_keeps_product_and_restores_orthogonality():
    """Re-orthogonalisation: same product, orthonormal U and B (§4.4)."""
    rng = np.random.default_rng(10)
    n, D, k = 50, 30, 6
    U = _orth(rng, n, k) + 1e-3 * rng.standard_normal((n, k))
    B = _orth(rng, D, k) + 1e-3 * rng.standard_normal((D, k))
    fac = _factor_from(U, np.linspace(3, 1, k), B)
    before = O.represented(fac)
    new = O.reorth(fac)
    assert np.linalg.norm(O.represented(new) - before) <= 1e-13 * np.linalg.norm(before)
    assert np.abs(new.U.T @ new.U - np.eye(k)).max() < 1e-13
    assert np.abs(new.B.T @ new.B - np.eye(k)).max() < 1e-13
    assert np.all(np.diff(new.sigma) <= 0)
    # an already-orthonormal factorisation keeps its singular values
    clean = _factor_from(_orth(rng, n, k), np.linspace(3, 1, k), _orth(rng, D, k))
    assert np.allclose(O.reorth(clean).sigma, np.linspace(3, 1, k), rtol=1e-13)


# ---------------------------------------------------------------- RoPE, bf16
def test_rope_closed_forms():
    hd, theta = 8, 10000.0
    rng = np.random.default_rng(11)
    X = rng.standard_normal((5, 2 * hd))
    # position 0 is the identity
    assert np.array_equal(O.rope(X, np.zeros(5), hd, theta), X)
    # a unit vector on feature j of head 1 turns into cos/sin on features j, j + hd/2
    for j in range(hd // 2):
        e = np.zeros((1, 2 * hd)); e[0, hd + j] = 1.0
        p = 37
        ang = p * theta ** (-2.0 * j / hd)
        out = O.rope(e, [p], hd, theta)
        exp = np.zeros(2 * hd); exp[hd + j] = math.cos(ang); exp[hd + j + hd // 2] = math.sin(ang)
        assert np.allclose(out[0], exp, atol=1e-15)
    # each pair keeps its norm; dot products depend only on the offset
    Y = O.rope(X, np.arange(5) * 11, hd, theta)
    for h in range(2):
        for j in range(hd // 2):
            a, b = h * hd + j, h * hd + j + hd // 2
            assert np.allclose(X[:, a] ** 2 + X[:, b] ** 2, Y[:, a] ** 2 + Y[:, b] ** 2)
    x, y = rng.standard_normal((1, hd)), rng.standard_normal((1, hd))
    d1 = O.rope(x, [100], hd, theta) @ O.rope(y, [90], hd, theta).T
    d2 = O.rope(x, [17], hd, theta) @ O.rope(y, [7], hd, theta).T
    assert abs(d1 - d2).max() < 1e-12


def test_reconstruct_turns_each_row_at_its_original_position():
    """Algorithm 3 / §3.2: keys are rotated at their original token position
    after the scatter, not at their compressed index. Planted unit rows on
    feature 0 of a head (whose pair angle is pos * theta**0 = pos radians for
    every theta) sit at shuffled positions; each must come out as
    (cos pos, sin pos) on features (0, d_h/2) of that head, a row at position 0
    must come out unturned, and two equal rows at positions a, b must have the
    dot product cos(b - a)."""
    rng = np.random.default_rng(31)
    hd, Hkv, theta = 8, 2, 500000.0
    D = Hkv * hd
    n_total = 40
    perm = rng.permutation(n_total)
    z = int(np.nonzero(perm == 0)[0][0])
    perm[z], perm[7] = perm[7], perm[z]          # position 0 sits at compressed index 7
    pos_c, pos_e = perm[:25], perm[25:]
    heads = rng.integers(0, Hkv, size=25)
    rows = np.zeros((25, D))
    rows[np.arange(25), heads * hd] = 1.0
    # a factor whose represented rows are exactly those unit rows
    U, s, Vt = np.linalg.svd(rows, full_matrices=False)
    k = int(np.count_nonzero(s > 1e-12))
    fac = O.Factor(U=U[:, :k], sigma=s[:k], B=Vt[:k].T, pos=pos_c.copy())
    X_e = rng.standard_normal((15, D))
    out = O.reconstruct(fac, X_e, pos_e, n_total, hd, apply_rope=True, theta=theta)
    for i, p in enumerate(pos_c):
        exp = np.zeros(D)
        exp[heads[i] * hd] = math.cos(p)
        exp[heads[i] * hd + hd // 2] = math.sin(p)
        assert np.allclose(out[p], exp, atol=1e-12), (i, p)
    i0 = int(np.nonzero(pos_c == 0)[0][0])
    assert np.allclose(out[0], rows[i0], atol=1e-12)
    same = [i for i in range(25) if heads[i] == heads[0]]
    a, b = pos_c[same[0]], pos_c[same[1]]
    assert abs(out[a] @ out[b] - math.cos(b - a)) < 1e-12
    # exact rows: norms of every (j, j + d_h/2) pair are kept at their positions
    for h in range(Hkv):
        for j in range(hd // 2):
            c0, c1 = h * hd + j, h * hd + j + hd // 2
            assert np.allclose(out[pos_e, c0] ** 2 + out[pos_e, c1] ** 2, X_e[:, c0] ** 2 + X_e[:, c1] ** 2)
    # turning at the compressed index instead would have been detected
    wrong = np.cos(np.arange(25)[pos_c != np.arange(25)])
    assert not np.allclose(out[pos_c[pos_c != np.arange(25)], heads[pos_c != np.arange(25)] * hd], wrong)


@pytest.mark.parametrize("T,b,n", [(256, 32, 1024), (1024, 64, 4096)])
def test_run_stream_reorth_schedule(monkeypatch, T, b, n):
    """§4.4: re-orthogonalisation runs each time the folded-row counter
    crosses a multiple of T (every T / b merges), and each call leaves the
    represented product unchanged while making B and U orthonormal."""
    calls = []
    real = O.iskv_oracle.reorth

    def counting(fac):
        new = real(fac)
        before, after = O.represented(fac), O.represented(new)
        calls.append((fac.folded, float(np.linalg.norm(after - before) / np.linalg.norm(before)),
                      float(np.abs(new.B.T @ new.B - np.eye(new.k)).max())))
        return new

    monkeypatch.setattr(O.iskv_oracle, "reorth", counting)
    merges = []
    X = synth.kv_stream(synth.StreamSpec(D=48, n=n, spectrum="exp4", noise_std=1e-3, seed=41))
    O.run_stream(X, b, 6, reorth_every_rows=T, callback=lambda t, f: merges.append(f.folded))
    assert [c[0] for c in calls] == list(range(T, n + 1, T))
    assert len(calls) == n // T and len(merges) == n // b
    for folded, drel, orth in calls:
        assert drel < 1e-12 and orth < 1e-12
    # T = 0 never re-orthogonalises; neither does the basis-only ablation
    calls.clear()
    O.run_stream(X[:4 * b], b, 6, reorth_every_rows=0)
    O.run_stream(X[:4 * b], b, 6, reorth_every_rows=b, sync=False)
    assert calls == []


def test_value_first_refit_resets_the_reorth_counter(monkeypatch):
    """§3.2 and §4.4: the value first refit is not a regular fold, so the
    folded-row counter restarts at zero after it, and the next
    re-orthogonalisation comes after T more folded rows."""
    X = synth.kv_stream(synth.StreamSpec(D=32, n=400, spectrum="invsqrt", noise_std=0.0, seed=42))
    fac = O.run_stream(X[:96], 16, 8, reorth_every_rows=64)
    assert fac.folded == 96
    fac = O.value_first_refit(fac, X[96:104], np.arange(96, 104), 8)
    assert fac.folded == 0
    calls = []
    real = O.iskv_oracle.reorth
    monkeypatch.setattr(O.iskv_oracle, "reorth", lambda f: (calls.append(f.folded), real(f))[1])
    O.run_stream(X[104:232], 16, 8, reorth_every_rows=64, fac=fac, pos0=104)
    assert calls == [64, 128]


def test_bf16_round_known_values():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38, 1e-40])
    got = O.bf16_round(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert got[0] == 1.0 and got[1] == 1.0
    assert got[2] == 1.0 + 2 ** -6           # tie between 1+2^-7 and 1+2^-6 -> even
    assert got[3] == 1.0
    assert got[4] == -2.5
    assert np.isfinite(got[5])


# ---------------------------------------------------------------- attention
def test_attend_special_cases():
    rng = np.random.default_rng(12)
    Bt, n, Hq, Hkv, dh = 2, 9, 8, 2, 4
    q = rng.standard_normal((Bt, Hq, dh))
    V = rng.standard_normal((Bt, n, Hkv, dh))
    # equal keys: the output is the mean of the values of the head's group
    K = np.broadcast_to(rng.standard_normal((1, 1, Hkv, dh)), (Bt, n, Hkv, dh)).copy()
    out = O.attend(q, K, V, 0.5)
    for h in range(Hq):
        assert np.allclose(out[:, h], V[:, :, h // (Hq // Hkv)].mean(axis=1), atol=1e-14)
    # a planted needle: one key along q with a huge logit picks its value row
    K = rng.standard_normal((Bt, n, Hkv, dh)) * 0.01
    K[:, 4, :, :] = 0.0
    for h in (0, 4):
        K[:, 4, h // 4, :] = 100.0 * q[:, h, :]
    out = O.attend(q, K, V, 1.0)
    assert np.allclose(out[:, 0], V[:, 4, 0], atol=1e-10)
    assert np.allclose(out[:, 4], V[:, 4, 1], atol=1e-10)


def _factor_v_case(seed, sync=True):
    """A small value path (D = 16 = 2 heads x 8, r = 4) folded from 24 rows,
    plus 6 exact rows, with the 30 positions shuffled between the two."""
    rng = np.random.default_rng(seed)
    D, dh, n_c, n_e = 16, 8, 24, 6
    X = rng.standard_normal((n_c, D)) @ np.diag(np.exp(-np.arange(D) / 3.0))
    perm = rng.permutation(n_c + n_e)
    pos_c, pos_e = np.sort(perm[:n_c]), perm[n_c:]
    fac = O.empty_factor(D, sync=sync)
    for s in range(0, n_c, 4):
        fac = O.merge(fac, X[s:s + 4], pos_c[s:s + 4], 4)
    X_e = rng.standard_normal((n_e, D))
    return fac, X_e, pos_e, n_c + n_e, dh


@pytest.mark.parametrize("sync", [True, False])
def test_attend_factor_v_equals_dense_on_reconstructed_values(sync):
    """Value attention on the factors = dense attention over the rebuilt value
    cache (the identity the factored decode rests on), also with the stale
    coordinates of the basis-only ablation."""
    fac, X_e, pos_e, n_total, dh = _factor_v_case(3, sync)
    rng = np.random.default_rng(4)
    Hq, Hkv = 4, 2
    q = rng.standard_normal((Hq, dh))
    K = rng.standard_normal((n_total, Hkv, dh))
    Vhat = O.reconstruct(fac, X_e, pos_e, n_total, dh, apply_rope=False)
    if not sync:  # the ablation keeps stale coordinates: the stored rows differ from U S B^T
        Vhat[fac.pos] = O.stored_rows(fac)
    dense = O.attend(q[None], K[None], Vhat.reshape(1, n_total, Hkv, dh), 0.3)[0]
    got = O.attend_factor_v(q, K, fac, X_e, pos_e, 0.3)
    assert np.allclose(got, dense, rtol=1e-12, atol=1e-12)


def test_attend_factor_v_special_cases():
    fac, X_e, pos_e, n_total, dh = _factor_v_case(5)
    Hq, Hkv = 4, 2
    rng = np.random.default_rng(6)
    q = rng.standard_normal((Hq, dh))
    C = fac.U * fac.sigma[None, :]
    # equal keys: every head returns the mean over all positions of its value slice
    K = np.broadcast_to(rng.standard_normal((1, Hkv, dh)), (n_total, Hkv, dh)).copy()
    got = O.attend_factor_v(q, K, fac, X_e, pos_e, 1.0)
    for h in range(Hq):
        g = h // 2
        want = (C.sum(axis=0) @ fac.B[g * dh:(g + 1) * dh].T + X_e[:, g * dh:(g + 1) * dh].sum(axis=0)) / n_total
        assert np.allclose(got[h], want, atol=1e-12)
    # a planted needle at a compressed position returns that row's rebuilt slice
    i = 7
    K = rng.standard_normal((n_total, Hkv, dh)) * 0.01
    K[fac.pos[i], 0] = 200.0 * q[0]
    got = O.attend_factor_v(q, K, fac, X_e, pos_e, 1.0)
    assert np.allclose(got[0], C[i] @ fac.B[:dh].T, atol=1e-9)
    # positions that do not partition the cache are refused
    with pytest.raises(ValueError):
        O.attend_factor_v(q, K[:-1], fac, X_e, pos_e, 1.0)


# ---------------------------------------------------------------- storage
def test_storage_accounting_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "storage_eq12.json")))
    be = g["breakeven"]
    assert O.breakeven_rows(be["D"], be["r"]) == be["rows"]
    for row in g["dense"]:
        tokens = row["input_tokens"] + row["generated"]
        got = O.dense_kv_bytes(tokens, g["layers"], g["D"], g["bytes_per_scalar"]) / 2 ** 30
        assert got == row["GiB"]
    # eq.(12) at the break-even: compressed payload below dense exactly from 147 rows
    D, r = be["D"], be["r"]
    assert O.persistent_bytes(147, 0, D, r, 2, 2) < 2 * 147 * D
    assert O.persistent_bytes(146, 0, D, r, 2, 2) >= 2 * 146 * D


def test_factor_drift_zero_without_truncation():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((24, 3)) @ rng.standard_normal((3, 10))
    fac = O.run_stream(X, 4, 6)
    assert abs(O.factor_drift(X, O.represented(fac), 6)) < 1e-12


# ---------------------------------------------------------------- tiny stream
def test_tiny_stream_fp32_tracks_fp64_and_near_fresh_svd():
    """The 32-merge tiny stream: fp32 and fp64 oracles agree; drift vs fresh SVD is small."""
    X = synth.kv_stream(synth.CONFIG_TINY)
    f64 = O.run_stream(X, 8, 8)
    f32 = O.run_stream(X, 8, 8, dtype=np.float32)
    R64 = O.represented(f64)
    R32 = (f32.U.astype(float) * f32.sigma.astype(float)) @ f32.B.astype(float).T
    assert np.linalg.norm(R64 - R32) / np.linalg.norm(R64) < 1e-4
    Xr, _ = O.fresh_truncated_svd(X, 8)
    rel_fresh = np.linalg.norm(X - Xr) / np.linalg.norm(X)
    drift = O.factor_drift(X, R64, 8)
    assert 0.0 <= drift < 0.5 * rel_fresh
    assert f64.n == 256 and f64.k == 8


# --------------------------------------------------------------------------- frozen basis
def test_fold_frozen_pins():
    """Frozen-basis fold (notes §6.4 / §8): rows inside span(B) are stored
    exactly; the new coordinates are the least-squares coordinates of F in B
    (numpy lstsq); the residual is orthogonal to B; old rows and B untouched."""
    rng = np.random.default_rng(31)
    D, k, n, b = 48, 7, 20, 5
    B, _ = np.linalg.qr(rng.standard_normal((D, k)))
    C = rng.standard_normal((n, k))
    pos = np.arange(n)
    # inside the span: F = Y B^T is stored exactly
    Y = rng.standard_normal((b, k))
    C2, pos2 = O.fold_frozen(C, B, pos, Y @ B.T, np.arange(n, n + b))
    assert np.array_equal(C2[:n], C)
    assert np.allclose(C2[n:], Y, atol=1e-12)
    assert np.array_equal(pos2, np.arange(n + b))
    assert np.allclose(C2[n:] @ B.T, Y @ B.T, atol=1e-12)
    # a general block: least-squares coordinates, residual orthogonal to B
    F = rng.standard_normal((b, D))
    C3, _ = O.fold_frozen(C, B, pos, F, np.arange(100, 100 + b))
    lsq = np.linalg.lstsq(B, F.T, rcond=None)[0].T
    assert np.allclose(C3[n:], lsq, atol=1e-12)
    assert np.abs((F - C3[n:] @ B.T) @ B).max() < 1e-12
    # a non-orthonormal basis is not what the fold assumes: its F B differs from lstsq
    B2 = B * np.linspace(1.0, 3.0, k)[None, :]
    C4, _ = O.fold_frozen(C, B2, pos, F, np.arange(b))
    assert not np.allclose(C4[n:], np.linalg.lstsq(B2, F.T, rcond=None)[0].T, atol=1e-6)


# --------------------------------------------------------------------------- 2-byte persistence
def test_persist_coords_bf16_pins():
    """Persistent 2-byte coordinates (notes §7.3): the stored C = U diag(sigma)
    becomes exactly bf16-representable (rounding again changes nothing), each
    entry moves by at most the bf16 unit roundoff (8 significant bits: 2^-8
    relative), sigma and B are untouched, and a column with sigma = 0 stays
    zero."""
    rng = np.random.default_rng(41)
    n, k, D = 30, 6, 20
    U, _ = np.linalg.qr(rng.standard_normal((n, k)))
    B, _ = np.linalg.qr(rng.standard_normal((D, k)))
    sigma = np.array([50.0, 7.0, 3.0, 1.0, 0.25, 0.0])
    fac = O.Factor(U=U, sigma=sigma, B=B, pos=np.arange(n))
    p = O.persist_coords_bf16(fac)
    C = fac.U * fac.sigma[None, :]
    Cp = p.U * p.sigma[None, :]
    # (U is held as C / sigma: multiplying back leaves fp64 rounding only)
    assert np.all(np.abs(O.bf16_round(Cp) - Cp) <= 1e-14 * np.abs(Cp))
    assert np.all(np.abs(Cp - C) <= 2.0 ** -8 * np.abs(C) + 1e-300)
    assert np.array_equal(p.sigma, fac.sigma) and np.array_equal(p.B, fac.B)
    assert np.all(p.U[:, 5] == 0)
    assert np.linalg.norm(O.represented(p) - O.represented(fac)) <= 2.0 ** -8 * np.linalg.norm(O.represented(fac))
    # a value half-way between two bf16 numbers rounds to the even one
    half = O.Factor(U=np.array([[1.0 + 2.0 ** -8]]), sigma=np.array([1.0]), B=np.eye(1), pos=np.arange(1))
    assert O.persist_coords_bf16(half).U[0, 0] == 1.0


def test_fp16_round_known_values():
    """IEEE binary16 (1 sign, 5 exponent, 10 fraction bits): ties go to the even
    fraction, 2^-24 is the smallest subnormal, 65504 = (2 - 2^-10) 2^15 the
    largest finite value; the guard stores larger magnitudes as +-65504 and
    reports them."""
    vals = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 1.0 + 2 ** -12, -2.5,
                     2.0 ** -24, 2.0 ** -26, 3 * 2.0 ** -25])
    got, over = O.fp16_round(vals)
    assert not over
    assert got[0] == 1.0 and got[1] == 1.0        # tie between 1 and 1 + 2^-10 -> even
    assert got[2] == 1.0 + 2 ** -9                # tie between 1 + 2^-10 and 1 + 2^-9 -> even
    assert got[3] == 1.0 and got[4] == -2.5
    assert got[5] == 2.0 ** -24 and got[6] == 0.0
    assert got[7] == 2.0 ** -23                   # subnormal tie -> even
    g, over = O.fp16_round(np.array([65504.0, -65504.0, 65500.0]))
    assert not over and g[0] == 65504.0 and g[1] == -65504.0 and g[2] == 65504.0
    for big in (65505.0, 65519.0, 65520.0, 1e6, 3e38):
        g, over = O.fp16_round(np.array([1.0, big, -big]))
        assert over and g[1] == 65504.0 and g[2] == -65504.0 and g[0] == 1.0
    g, over = O.fp16_round(np.array([np.nan, 2.0]))
    assert not over and np.isnan(g[0]) and g[1] == 2.0
    # without the guard a value past 65520 would round to an infinity
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(65520.0).astype(np.float16))


def test_persist_coords_fp16_pins():
    """Persistent fp16 coordinates (notes §7.3): the stored C = U diag(sigma) is
    exactly half-representable, entries move by at most 2^-11 relative (11
    significant bits) above the subnormal range, sigma and B are untouched; a
    coordinate above 65504 in magnitude is saturated, the factor stays finite
    and flagged, and the flag is sticky through later merges and
    re-orthogonalisations of a stream."""
    rng = np.random.default_rng(43)
    n, k, D = 30, 6, 20
    U, _ = np.linalg.qr(rng.standard_normal((n, k)))
    B, _ = np.linalg.qr(rng.standard_normal((D, k)))
    sigma = np.array([900.0, 70.0, 3.0, 1.0, 0.25, 0.0])
    fac = O.Factor(U=U, sigma=sigma, B=B, pos=np.arange(n))
    p = O.persist_coords_fp16(fac)
    C = fac.U * fac.sigma[None, :]
    Cp = p.U * p.sigma[None, :]
    assert not p.fp16_overflow
    assert np.all(np.abs(O.fp16_round(Cp)[0] - Cp) <= 1e-14 * np.abs(Cp))
    normal = np.abs(C) >= 2.0 ** -14
    assert np.all(np.abs(Cp - C)[normal] <= 2.0 ** -11 * np.abs(C)[normal])
    assert np.all(np.abs(Cp - C)[~normal] <= 2.0 ** -25)
    assert np.array_equal(p.sigma, fac.sigma) and np.array_equal(p.B, fac.B)
    assert np.all(p.U[:, 5] == 0)
    # sigma_1 = 2e5 on a column whose largest entry is ~0.6: C passes 65504
    big = O.Factor(U=U, sigma=np.array([2e5, 70.0, 3.0, 1.0, 0.25, 0.0]), B=B, pos=np.arange(n))
    pb = O.persist_coords_fp16(big)
    Cb = pb.U * pb.sigma[None, :]
    assert pb.fp16_overflow and np.all(np.isfinite(Cb))
    hit = np.abs(U[:, 0] * 2e5) > 65504.0
    # (U is held as C / sigma: multiplying back leaves fp64 rounding only)
    assert hit.any() and np.allclose(np.abs(Cb[hit, 0]), 65504.0, rtol=1e-14, atol=0)
    assert np.all(np.sign(Cb[hit, 0]) == np.sign(U[hit, 0]))
    # a stream of large rows: the fp16 path saturates and reports, stays finite
    # and keeps reporting; bf16 (8 exponent bits) holds the same values
    X = synth.kv_stream(synth.StreamSpec(D=64, n=96, spectrum="exp4", noise_std=1e-3, seed=44)) * 3e4
    f16 = O.run_stream(X, 16, 8, reorth_every_rows=32, persist_fp16=True)
    assert f16.fp16_overflow and np.all(np.isfinite(f16.U * f16.sigma[None, :]))
    assert np.abs(f16.U * f16.sigma[None, :]).max() <= 65504.0 * (1 + 1e-12)
    f16b = O.run_stream(X, 16, 8, reorth_every_rows=32, persist_bf16=True)
    assert not f16b.fp16_overflow and np.abs(f16b.U * f16b.sigma[None, :]).max() > 65504.0
    small = O.run_stream(X / 3e4, 16, 8, reorth_every_rows=32, persist_fp16=True)
    assert not small.fp16_overflow
    with pytest.raises(ValueError):
        O.run_stream(X, 16, 8, persist_bf16=True, persist_fp16=True)


# --------------------------------------------------------------------------- prompt protection
def test_anomaly_scores_and_protect_pins():
    """Algorithm 1 (notes §3.1): a block of equal keys scores 1, one
    key opposite to the rest gives that key's cosine with the mean (closed
    form), the suffix (last 4 blocks + tail) is never scored and always kept,
    a head keeps its lowest blocks (ties: lower index), P_V dilates P_K by 32
    positions (brute force) and W_V is the last 128 positions."""
    Hkv, dh, blk = 2, 4, 8
    L = 8 * 9 + 3                       # 9 whole blocks + a tail of 3: 5 scored blocks
    rng = np.random.default_rng(51)
    K = np.tile(rng.standard_normal((1, Hkv * dh)), (L, 1))   # every key equal: every score 1
    sc, s0 = O.anomaly_block_scores(K, Hkv, dh)
    assert sc.shape == (2, 5) and s0 == 40 and np.allclose(sc, 1.0)
    # block 2, head 1: seven keys e and one key -e -> mean 6e/8, cosine of the odd key = -1
    e = np.array([1.0, 0.0, 0.0, 0.0])
    K[16:24, dh:2 * dh] = e
    K[19, dh:2 * dh] = -e
    # block 4, head 0: keys e and one key orthogonal: mean (7e + f)/8, min cosine = 1/sqrt(50)
    f = np.array([0.0, 1.0, 0.0, 0.0])
    K[32:40, :dh] = e
    K[35, :dh] = f
    sc, _ = O.anomaly_block_scores(K, Hkv, dh)
    assert abs(sc[1, 2] + 1.0) < 1e-12
    assert abs(sc[0, 4] - 1.0 / np.sqrt(50.0)) < 1e-12
    pk, pv, wv = O.prompt_protect(K, Hkv, dh, per_head=1)
    expect = np.zeros(L, dtype=bool)
    expect[16:24] = True                # head 1's lowest block
    expect[32:40] = True                # head 0's lowest block
    expect[40:] = True                  # suffix
    assert np.array_equal(pk, expect)
    brute = np.array([any(pk[q] for q in range(max(0, p - 32), min(L, p + 33))) for p in range(L)])
    assert np.array_equal(pv, brute)
    assert np.array_equal(wv, np.arange(L) >= L - 128)
    # ties: all scores equal -> the lowest block indices; fewer blocks than per_head -> all
    pk2, _, _ = O.prompt_protect(np.tile(K[:1], (L, 1)), Hkv, dh, per_head=2)
    assert np.array_equal(np.nonzero(pk2[:40])[0], np.arange(16))
    pk3, _, _ = O.prompt_protect(K, Hkv, dh, per_head=128)
    assert pk3.all()
    # a prompt shorter than the suffix: nothing scored, everything protected
    sc4, s4 = O.anomaly_block_scores(K[:30], Hkv, dh)
    assert sc4.shape == (2, 0) and s4 == 0
    assert O.prompt_protect(K[:30], Hkv, dh)[0].all()


def _orthonormal(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


def test_truncated_factor_and_prefill_init_pins():
    """Algorithm 1 (notes §3.1): each path's factor covers exactly its
    non-exact rows (positions saved in order; the exact rows, here planted
    with huge values, never reach it), a non-exact part of rank <= r is
    reproduced exactly, and truncation keeps the r largest of known singular
    values with error^2 = the sum of the rest (Eckart-Young, closed form)."""
    rng = np.random.default_rng(81)
    Hkv, dh = 2, 8
    D, L = Hkv * dh, 8 * 40
    K_rot = rng.standard_normal((L, D))
    pk, pv, wv = O.prompt_protect(K_rot, Hkv, dh, per_head=3)
    E_K, E_V = pk, pv | wv
    assert 0 < (~E_K).sum() and 0 < (~E_V).sum() < (~E_K).sum()
    K_pre = 1e6 * rng.standard_normal((L, D))
    V = 1e6 * rng.standard_normal((L, D))
    K_pre[~E_K] = rng.standard_normal(((~E_K).sum(), 3)) @ rng.standard_normal((3, D))
    V[~E_V] = rng.standard_normal(((~E_V).sum(), 4)) @ rng.standard_normal((4, D))
    fK, fV, eK, eV = O.prefill_init(K_pre, K_rot, V, Hkv, dh, r_K=5, r_V=4, per_head=3)
    assert np.array_equal(eK, E_K) and np.array_equal(eV, E_V)
    assert np.array_equal(fK.pos, np.nonzero(~E_K)[0]) and np.array_equal(fV.pos, np.nonzero(~E_V)[0])
    for f, X in ((fK, K_pre[~E_K]), (fV, V[~E_V])):
        assert np.abs(O.represented(f) - X).max() < 1e-10 * np.abs(X).max()
        assert np.abs(f.B.T @ f.B - np.eye(f.k)).max() < 1e-12
    # known singular values 5, 4, 3, 2, 1: rank 2 keeps 5 and 4, error^2 = 9 + 4 + 1
    sv = np.array([5.0, 4.0, 3.0, 2.0, 1.0])
    Q1, Q2 = _orthonormal(rng, 40, 5), _orthonormal(rng, D, 5)
    X = (Q1 * sv) @ Q2.T
    f = O.truncated_factor(X, np.arange(100, 140), 2)
    assert np.allclose(f.sigma, [5.0, 4.0], atol=1e-12)
    assert abs(np.linalg.norm(X - O.represented(f)) ** 2 - 14.0) < 1e-10
    assert np.allclose(np.abs(f.B.T @ Q2[:, :2]), np.eye(2), atol=1e-12)
    assert np.array_equal(f.pos, np.arange(100, 140))
    assert O.truncated_factor(np.zeros((0, D)), [], 4).n == 0


def test_value_first_refit_pins():
    """§3.2 value first refit: the fresh SVD of [reconstructed history; rows].
    History rows 5 e1 and 4 e2, a new row 3 e3, rank 2: keeps 5 and 4 and
    loses the new row (error^2 = 9); with the new row 6 e3 the refit keeps
    6 and 5 and drops an old direction (error^2 = 16); positions: the
    history's, then the new rows'. Rank <= r: exact."""
    D = 6
    e = np.eye(D)
    hist = O.truncated_factor(np.stack([5 * e[0], 4 * e[1]]), [7, 9], 2)
    for new, keep, err2 in ((3.0, [5.0, 4.0], 9.0), (6.0, [6.0, 5.0], 16.0)):
        f = O.value_first_refit(hist, (new * e[2])[None, :], [30], 2)
        assert np.allclose(f.sigma, keep, atol=1e-12)
        stacked = np.stack([5 * e[0], 4 * e[1], new * e[2]])
        assert abs(np.linalg.norm(stacked - O.represented(f)) ** 2 - err2) < 1e-10
        assert list(f.pos) == [7, 9, 30]
    f = O.value_first_refit(hist, np.stack([e[0] + e[1], 2 * e[1]]), [30, 31], 3)
    assert np.abs(O.represented(f) - np.stack([5 * e[0], 4 * e[1], e[0] + e[1], 2 * e[1]])).max() < 1e-12
