"""The core eigensolver on its own (iS-KV notes §4.2: SVD of the small core),
checked against the defining properties of a symmetric eigendecomposition:
A V = V Lambda, V^T V = I, eigenvalues equal to LAPACK's (numpy.linalg.eigh)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import synth  # noqa: E402


@pytest.fixture(scope="module")
def path():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_rank_kv_amd as K
    p = K.IsvdPath(D=1024, r_max=256, b_max=64, n_cap=64, device="cuda")
    yield p
    p.close()


def core_of_stream(kind, r, b, n, seed=0):
    X = synth.kv_stream(synth.StreamSpec(D=1024, n=n + b, spectrum=kind, noise_std=0.0, seed=seed))
    fac = O.run_stream(X[:n], b, r)
    d = {}
    O.merge(fac, X[n:n + b], np.arange(n, n + b), r, diag=d)
    Z = d["Z"]
    return Z.T @ Z


def matrices():
    rng = np.random.default_rng(0)
    out = {}
    out["steady_kstream_n8192"] = core_of_stream("exp40+0.01", 256, 32, 8192)
    out["early_kstream_n256"] = core_of_stream("exp40+0.01", 256, 32, 256)
    out["vstream_n2048"] = core_of_stream("invsqrt", 256, 32, 2048, seed=1)
    Q = np.linalg.qr(rng.standard_normal((40, 40)))[0]
    out["dense_spd_40"] = Q @ np.diag(np.linspace(1, 5, 40)) @ Q.T
    out["identity_12"] = np.eye(12)
    A = np.diag([3.0, 3.0, 3.0, 1.0, 1.0, 0.5])
    A[0, 1] = A[1, 0] = 0.3
    A[3, 4] = A[4, 3] = 1e-3
    out["ties_6"] = A
    out["one"] = np.array([[2.5]])
    out["zero_4"] = np.zeros((4, 4))
    return out


@pytest.mark.parametrize("name", list(matrices().keys()))
def test_sym_eig(path, name):
    A = matrices()[name]
    m = A.shape[0]
    lam, V = path.sym_eig(torch.from_numpy(np.ascontiguousarray(A)).cuda())
    torch.cuda.synchronize()
    lam = lam.cpu().numpy()
    V = V.cpu().numpy()
    st = path.state()
    ref = np.linalg.eigvalsh(A)[::-1]
    scale = max(np.abs(ref).max(), 1e-300)
    print(f"{name}: m={m} flags={st[11]} steps={st[12]} lam err {np.abs(lam - ref).max() / scale:.2e} "
          f"orth {np.abs(V.T @ V - np.eye(m)).max():.2e} resid {np.linalg.norm(A @ V - V * lam) / max(np.linalg.norm(A), 1e-300):.2e}")
    assert np.all(np.diff(lam) <= 1e-12 * scale)
    assert np.abs(lam - ref).max() <= 1e-10 * scale
    assert np.abs(V.T @ V - np.eye(m)).max() < 1e-10
    assert np.linalg.norm(A @ V - V * lam) <= 1e-10 * max(np.linalg.norm(A), 1e-300)


@pytest.fixture()
def big_path():
    """A fresh handle per case (the status bits are sticky)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_rank_kv_amd as K
    p = K.IsvdPath(D=1024, r_max=512, b_max=64, n_cap=64, device="cuda")
    yield p
    p.close()


def big_matrices():
    rng = np.random.default_rng(3)
    out = {}
    for m, kind in ((576, "floor"), (400, "clusters"), (333, "floor")):
        Q = np.linalg.qr(rng.standard_normal((m, m)))[0]
        if kind == "floor":      # squared K-stream spectrum: hundreds of nearly equal values
            lam = (np.exp(-np.arange(m) / 40.0) + 0.01) ** 2
        else:                    # exact ties in groups of 8 plus a spread
            lam = np.repeat(np.linspace(1.0, 0.01, m // 8), 8)
        out[f"dense_{kind}_{m}"] = (Q * lam) @ Q.T
    return out


@pytest.mark.parametrize("name", list(big_matrices().keys()))
def test_sym_eig_dense_large(big_path, name):
    """Dense cores above 288 (the refinement cannot converge from a dense start)
    are finished by the block-Jacobi fallback: LAPACK's eigenvalues to 1e-10,
    orthonormal eigenvectors, A V = V Lambda."""
    A = big_matrices()[name]
    m = A.shape[0]
    lam, V = big_path.sym_eig(torch.from_numpy(np.ascontiguousarray(A)).cuda())
    torch.cuda.synchronize()
    lam = lam.cpu().numpy()
    V = V.cpu().numpy()
    st = big_path.state()
    ref = np.linalg.eigvalsh(A)[::-1]
    scale = np.abs(ref).max()
    Sv = V.T @ A @ V
    dg = np.abs(np.diag(Sv))
    den = np.maximum(np.sqrt(np.outer(dg, dg)), 0.01 * dg.max())
    off = np.abs(Sv - np.diag(np.diag(Sv))) / den
    print(f"{name}: max scaled coupling of V^T A V {off.max():.2e}")
    print(f"{name}: flags={st[11]} sweeps={st[7]} status={st[4]} lam err {np.abs(lam - ref).max() / scale:.2e} "
          f"orth {np.abs(V.T @ V - np.eye(m)).max():.2e} resid {np.linalg.norm(A @ V - V * lam) / np.linalg.norm(A):.2e}")
    assert st[4] == 0
    assert np.abs(lam - ref).max() <= 1e-10 * scale
    assert np.abs(V.T @ V - np.eye(m)).max() < 1e-10
    assert np.linalg.norm(A @ V - V * lam) <= 1e-10 * np.linalg.norm(A)
