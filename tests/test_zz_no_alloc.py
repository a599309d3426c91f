"""decode_attend_noalloc: the no-allocation form of decode_attend (for
callers that cannot allocate device memory) against decode_attend itself,
through the C ABI: two calls in a row, the second smaller, each equal to
decode_attend's output on the same inputs (same kernels, so bit for bit), and
within the attention bar (2e-2) of the oracle; a call beyond the fixed
scratch is refused before anything runs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import online_rank_kv_amd as mod
    return mod


def _case(batch, n, hq, hkv, seed):
    rng = np.random.default_rng(seed)
    Kc = torch.from_numpy(rng.standard_normal((batch, n, hkv, 128)).astype(np.float32)).cuda().bfloat16()
    Vc = torch.from_numpy(rng.standard_normal((batch, n, hkv, 128)).astype(np.float32)).cuda().bfloat16()
    q = torch.from_numpy(rng.standard_normal((batch, hq, 128)).astype(np.float32)).cuda().bfloat16()
    return q, Kc, Vc


def test_noalloc_attention_matches_decode_attend(K):
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    for batch, n, hq, hkv in ((2, 20000, 32, 8), (1, 1000, 32, 8)):
        q, Kc, Vc = _case(batch, n, hq, hkv, 100 + n)
        scale = 128 ** -0.5
        ref = torch.empty((batch, hq, 128), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(K.decode_attend_workspace_bytes(batch, n, hq, 128), dtype=torch.uint8, device="cuda")
        K.decode_attend(q, Kc, Vc, batch, n, hq, hkv, 128, scale, ref, ws)
        got = torch.full((batch, hq, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        K.decode_attend_noalloc(q, Kc, Vc, batch, n, hq, hkv, 128, scale, got, stream=stream)
        stream.synchronize()
        assert torch.equal(got, ref), (batch, n)
        if n <= 1000:
            oref = O.attend(q.float().cpu().numpy(), Kc.float().cpu().numpy(), Vc.float().cpu().numpy(), scale)
            assert np.abs(got.float().cpu().numpy() - oref).max() < 2e-2
    # beyond the fixed scratch (32 heads x 1563 splits x 520 bytes > 8 MiB): refused, output untouched
    q, Kc, Vc = _case(1, 200_000, 32, 8, 7)
    out = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(K.IskvError) as e:
        K.decode_attend_noalloc(q, Kc, Vc, 1, 200_000, 32, 8, 128, 0.1, out)
    assert e.value.code == -3
    torch.cuda.synchronize()
    assert not out.any()
