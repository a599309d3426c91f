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
