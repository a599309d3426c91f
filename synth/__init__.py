"""Seeded synthetic KV streams shared by the oracle's tests and the GPU path's tests/bench.

This module holds no arithmetic of the compression method itself: it only draws
random numbers in a fixed order and shapes them like the pages' workloads
(Llama-8B-like KV rows: 8 KV heads x 128 = 1024 features, low-rank-plus-noise
spectra). Both the CPU oracle and the GPU path consume the identical fp32 rows
it returns.

Recipe (one stream): draw, in this order and from one ``numpy.random.Generator``
seeded with ``seed``,
  1. a Haar-random D x D orthonormal basis O (QR of a Gaussian matrix, columns
     sign-fixed by the sign of R's diagonal, as in Mezzadri's construction);
  2. i.i.d. N(0, 1) coordinates Zc of shape n x D;
  3. optional i.i.d. N(0, noise_std^2) noise of shape n x D;
and return X = (Zc * sigma) @ O^T + noise cast to float32, where sigma_i is the
stream's population spectrum, index i = 0 .. D-1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "haar_orthonormal",
    "spectrum",
    "kv_stream",
    "StreamSpec",
    "CONFIG_TINY",
    "CONFIG_KSTREAM",
    "CONFIG_KV_K",
    "CONFIG_KV_V",
    "protected_prompt_rows",
    "bf16_queries",
    "DeviceStreams",
]


def haar_orthonormal(rng: np.random.Generator, d: int) -> np.ndarray:
    """Haar-distributed d x d orthonormal matrix (QR of a Gaussian, sign-fixed)."""
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return q * s[None, :]


def spectrum(kind: str, d: int) -> np.ndarray:
    """Population spectra of the synthetic workloads, index i = 0 .. d-1.

    ``"exp4"``:      exp(-i/4)              (tiny stream)
    ``"exp40+0.01"``: exp(-i/40) + 0.01     (key stream)
    ``"invsqrt"``:   (1 + i) ** -0.5        (value stream)
    """
    i = np.arange(d, dtype=np.float64)
    if kind == "exp4":
        return np.exp(-i / 4.0)
    if kind == "exp40+0.01":
        return np.exp(-i / 40.0) + 0.01
    if kind == "invsqrt":
        return (1.0 + i) ** -0.5
    raise ValueError(f"unknown spectrum {kind!r}")


@dataclass(frozen=True)
class StreamSpec:
    D: int
    n: int
    spectrum: str
    noise_std: float
    seed: int


# Tiny stream: D=64, n=256, sigma_i = exp(-i/4), noise std 1e-3, seed 0.
CONFIG_TINY = StreamSpec(D=64, n=256, spectrum="exp4", noise_std=1e-3, seed=0)
# Llama-8B-shaped key stream: D = 8 x 128, 16384 rows, exp(-i/40)+0.01, seed 0.
CONFIG_KSTREAM = StreamSpec(D=1024, n=16384, spectrum="exp40+0.01", noise_std=0.0, seed=0)
# K and V together: K as above (seed 0), V with (1+i)^-1/2 (seed 1).
CONFIG_KV_K = CONFIG_KSTREAM
CONFIG_KV_V = StreamSpec(D=1024, n=16384, spectrum="invsqrt", noise_std=0.0, seed=1)


def kv_stream(spec: StreamSpec, n: int | None = None) -> np.ndarray:
    """Rows of one synthetic KV stream as float32, shape (n, D).

    ``n`` may be smaller than ``spec.n`` to take a prefix; the prefix is
    identical to the first rows of the full stream (coordinates are drawn row
    by row after the basis).
    """
    n_full = spec.n
    n = n_full if n is None else int(n)
    if n > n_full:
        raise ValueError("prefix longer than the stream")
    rng = np.random.default_rng(spec.seed)
    O = haar_orthonormal(rng, spec.D)
    zc = rng.standard_normal((n, spec.D))
    sig = spectrum(spec.spectrum, spec.D)
    x = (zc * sig[None, :]) @ O.T
    if spec.noise_std > 0.0:
        x = x + spec.noise_std * rng.standard_normal((n, spec.D))
    return x.astype(np.float32)


def protected_prompt_rows(prompt_len: int, block: int, frac: float, suffix_blocks: int,
                          v_radius: int, seed: int):
    """Seeded stand-in for the prompt protection sets.

    A random ``frac`` of the ``block``-token prompt blocks, plus the last
    ``suffix_blocks`` whole blocks and the partial tail, form the protected key
    positions; protected value positions are every prompt position within
    ``v_radius`` of a protected key position. Returns two sorted int32 arrays.
    """
    rng = np.random.default_rng(seed)
    nblk_full = prompt_len // block
    tail_start = nblk_full * block
    n_pick = int(math.floor(frac * nblk_full + 0.5))
    picked = rng.choice(nblk_full, size=n_pick, replace=False) if n_pick > 0 else np.array([], int)
    kmask = np.zeros(prompt_len, dtype=bool)
    for b in picked:
        kmask[b * block:(b + 1) * block] = True
    suf0 = max(0, (nblk_full - suffix_blocks) * block)
    kmask[suf0:] = True
    kmask[tail_start:] = True
    kpos = np.nonzero(kmask)[0]
    vmask = np.zeros(prompt_len, dtype=bool)
    for p in kpos:
        vmask[max(0, p - v_radius):min(prompt_len, p + v_radius + 1)] = True
    vpos = np.nonzero(vmask)[0]
    return kpos.astype(np.int32), vpos.astype(np.int32)


def bf16_queries(batch: int, hq: int, dh: int, seed: int) -> np.ndarray:
    """N(0, 1) decode queries rounded to bf16, returned as the uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, hq, dh)).astype(np.float32)
    u = q.view(np.uint32).astype(np.uint64)
    # round-to-nearest-even to the upper 16 bits
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


class DeviceStreams:
    """Many independent streams drawn on the GPU (the many-path workload: every
    (sequence, layer, K/V) path is its own stream).

    Path z < n_k uses the key spectrum (exp(-i/40) + 0.01), the others the
    value spectrum ((1+i)^-1/2); each kind has one Haar basis drawn on the host
    as in ``kv_stream`` (seeds ``seed`` and ``seed + 1``), and the coordinates
    of every path are i.i.d. N(0, 1) from one seeded device generator, drawn
    block by block in call order. ``rows(c)`` returns the next c rows of every
    path as a float32 tensor [paths, c, D] on ``device``.
    """

    def __init__(self, paths: int, n_k: int, D: int, seed: int, device):
        import torch
        self.paths, self.n_k, self.D = paths, n_k, D
        self.device = torch.device(device)
        bases, sigmas = [], []
        for kind, sd in (("exp40+0.01", seed), ("invsqrt", seed + 1)):
            O = haar_orthonormal(np.random.default_rng(sd), D)
            bases.append(torch.from_numpy(np.ascontiguousarray(O.T)).to(self.device, torch.float32))
            sigmas.append(torch.from_numpy(spectrum(kind, D)).to(self.device, torch.float32))
        self.OT, self.sig = bases, sigmas
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(seed + 2)

    def rows(self, c: int):
        import torch
        z = torch.randn((self.paths, c, self.D), generator=self.gen, device=self.device, dtype=torch.float32)
        out = torch.empty_like(z)
        nk = self.n_k
        if nk > 0:
            out[:nk] = torch.matmul(z[:nk] * self.sig[0], self.OT[0])
        if nk < self.paths:
            out[nk:] = torch.matmul(z[nk:] * self.sig[1], self.OT[1])
        return out


def prompt_keys(L: int, Hkv: int, dh: int, seed: int) -> np.ndarray:
    """Post-RoPE prompt keys (fp32 [L, Hkv * dh]) for the anomaly-score rule:
    N(0, 1) entries, and in every fifth 8-token block the token at offset 2
    turned against its block and doubled (a planted anomaly)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, Hkv * dh)).astype(np.float32)
    for j in range(0, L // 8, 5):
        k[8 * j + 2] = -2.0 * k[8 * j + 2]
    return k
