"""Python binding of the gfx950 iS-KV hot path (libiskv.so).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/iskv.h``. PyTorch supplies device memory and
streams. The names follow the C entry points (``isvd_init``,
``isvd_merge_block``, ``isvd_reorth``, ``isvd_query``, ``kv_reconstruct``,
``decode_attend`` and the ``iskv_window_*`` calls); ``IsvdPath`` and
``ExactWindow`` own the torch tensors that back one handle.

Importing the package loads the shared library and fails loudly when it has
not been built (``python -m online_rank_kv_amd.build`` or
``__graft_entry__.build()``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LIB_PATH", "lib", "IskvError", "IskvConfig", "ISKV_NO_COORD_SYNC", "ISKV_NO_GRAPH", "ISKV_FROZEN_BASIS",
    "ISKV_BF16_COORDS", "ISKV_FP16_COORDS", "ISKV_DEV_FP16_OVERFLOW", "isvd_refit_workspace_bytes", "isvd_refit", "isvd_value_first_refit_workspace_bytes",
    "isvd_value_first_refit", "iskv_prompt_split_workspace_bytes", "iskv_prompt_split", "prompt_split",
    "prefill_init", "iskv_prompt_protect_workspace_bytes", "iskv_prompt_protect", "prompt_protect",
    "ISKV_OUT_BF16", "isvd_set_mode",
    "ISKV_OUT_FP32", "ISKV_DEV_NONFINITE", "ISKV_DEV_NOCONV", "EXPORTED_SYMBOLS",
    "isvd_workspace_bytes", "isvd_init", "isvd_merge_block", "isvd_reorth", "isvd_query", "isvd_copy",
    "isvd_rows", "isvd_destroy", "isvd_query_state", "isvd_sym_eig", "kv_reconstruct", "kv_reconstruct_batched",
    "kv_scatter_exact",
    "decode_attend_workspace_bytes", "decode_attend", "decode_attend_noalloc", "decode_attend_fv_workspace_bytes",
    "decode_attend_fv", "iskv_window_rows", "iskv_window_init", "iskv_window_protect",
    "iskv_window_append", "iskv_window_exact", "iskv_window_destroy", "iskv_strerror",
    "iskv_window_append_batched", "isvd_merge_block_batched", "isvd_set_timing", "isvd_stage_times", "MERGE_STAGES", "IsvdPath", "IsvdBatch", "ExactWindow",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libiskv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m online_rank_kv_amd.build)")

lib = ctypes.CDLL(LIB_PATH)

ISKV_NO_COORD_SYNC = 1
ISKV_NO_GRAPH = 2
ISKV_FROZEN_BASIS = 4
ISKV_BF16_COORDS = 8
ISKV_FP16_COORDS = 16
ISKV_OUT_BF16 = 0
ISKV_OUT_FP32 = 1
ISKV_DEV_NONFINITE = 1
ISKV_DEV_NOCONV = 2
ISKV_DEV_FP16_OVERFLOW = 4

EXPORTED_SYMBOLS = (
    "isvd_workspace_bytes", "isvd_init", "isvd_merge_block", "isvd_reorth", "isvd_query",
    "isvd_rows", "isvd_destroy", "kv_reconstruct", "kv_reconstruct_batched", "decode_attend_workspace_bytes",
    "decode_attend", "iskv_window_rows", "iskv_window_init", "iskv_window_protect",
    "iskv_window_append", "iskv_window_exact", "iskv_window_destroy", "iskv_strerror",
    "isvd_query_state", "isvd_sym_eig", "kv_scatter_exact", "isvd_merge_block_batched",
    "isvd_set_timing", "isvd_stage_times", "iskv_window_append_batched",
    "decode_attend_fv_workspace_bytes", "decode_attend_fv", "isvd_set_mode",
    "iskv_prompt_protect_workspace_bytes", "iskv_prompt_protect", "isvd_refit_workspace_bytes", "isvd_refit",
    "isvd_value_first_refit_workspace_bytes", "isvd_value_first_refit", "iskv_prompt_split_workspace_bytes",
    "iskv_prompt_split", "decode_attend_noalloc", "isvd_copy",
)


class IskvConfig(ctypes.Structure):
    _fields_ = [
        ("D", ctypes.c_int32),
        ("r_max", ctypes.c_int32),
        ("b_max", ctypes.c_int32),
        ("n_cap", ctypes.c_int32),
        ("reorth_every_rows", ctypes.c_int32),
        ("resid_rel_tol", ctypes.c_float),
        ("flags", ctypes.c_int32),
    ]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_pi32 = ctypes.POINTER(ctypes.c_int32)

lib.iskv_strerror.restype = ctypes.c_char_p
lib.iskv_strerror.argtypes = [ctypes.c_int]
lib.isvd_workspace_bytes.restype = ctypes.c_size_t
lib.isvd_workspace_bytes.argtypes = [ctypes.POINTER(IskvConfig)]
lib.isvd_init.restype = ctypes.c_int
lib.isvd_init.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(IskvConfig), _vp, _vp, _vp, _vp, _vp,
                          ctypes.c_size_t, _vp]
lib.isvd_merge_block.restype = ctypes.c_int
lib.isvd_merge_block.argtypes = [_vp, _vp, _vp, _i32]
lib.isvd_merge_block_batched.restype = ctypes.c_int
lib.isvd_merge_block_batched.argtypes = [ctypes.POINTER(_vp), _i32, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                         _i32]
lib.isvd_reorth.restype = ctypes.c_int
lib.isvd_reorth.argtypes = [_vp]
lib.isvd_copy.argtypes = [_vp, _vp]
lib.isvd_set_mode.restype = ctypes.c_int
lib.isvd_set_mode.argtypes = [_vp, _i32]
lib.isvd_refit_workspace_bytes.restype = ctypes.c_size_t
lib.isvd_refit_workspace_bytes.argtypes = [_vp]
lib.isvd_refit.restype = ctypes.c_int
lib.isvd_refit.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, ctypes.c_size_t]
lib.isvd_value_first_refit_workspace_bytes.restype = ctypes.c_size_t
lib.isvd_value_first_refit_workspace_bytes.argtypes = [_vp]
lib.isvd_value_first_refit.restype = ctypes.c_int
lib.isvd_value_first_refit.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, ctypes.c_size_t]
lib.iskv_prompt_split_workspace_bytes.restype = ctypes.c_size_t
lib.iskv_prompt_split_workspace_bytes.argtypes = [_i32]
lib.iskv_prompt_split.restype = ctypes.c_int
lib.iskv_prompt_split.argtypes = [_vp, _vp, _i32, _i32, ctypes.c_uint32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
lib.iskv_prompt_protect_workspace_bytes.restype = ctypes.c_size_t
lib.iskv_prompt_protect_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
lib.iskv_prompt_protect.restype = ctypes.c_int
lib.iskv_prompt_protect.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]
lib.isvd_query.restype = ctypes.c_int
lib.isvd_query.argtypes = [_vp, _pi32, _pi32, _pi32]
lib.isvd_query_state.restype = ctypes.c_int
lib.isvd_query_state.argtypes = [_vp, _pi32, _i32]
lib.isvd_sym_eig.restype = ctypes.c_int
lib.isvd_sym_eig.argtypes = [_vp, _vp, _i32, _vp, _vp]
lib.isvd_set_timing.restype = ctypes.c_int
lib.isvd_set_timing.argtypes = [_vp, _i32]
lib.isvd_stage_times.restype = ctypes.c_int
lib.isvd_stage_times.argtypes = [_vp, ctypes.POINTER(ctypes.c_float), _i32]
lib.isvd_rows.restype = _i32
lib.isvd_rows.argtypes = [_vp]
lib.isvd_destroy.restype = None
lib.isvd_destroy.argtypes = [_vp]
lib.kv_reconstruct.restype = ctypes.c_int
lib.kv_reconstruct.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _i32, _vp]
lib.kv_reconstruct_batched.restype = ctypes.c_int
lib.kv_reconstruct_batched.argtypes = [ctypes.POINTER(_vp), _i32, ctypes.POINTER(_vp), ctypes.POINTER(_i32),
                                       ctypes.POINTER(_i32), _i32, ctypes.c_float, _vp]
lib.kv_scatter_exact.restype = ctypes.c_int
lib.kv_scatter_exact.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _i32, _vp]
lib.decode_attend_workspace_bytes.restype = ctypes.c_size_t
lib.decode_attend_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
lib.decode_attend.restype = ctypes.c_int
lib.decode_attend.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _vp,
                              ctypes.c_size_t, _vp]
lib.decode_attend_noalloc.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _vp]
lib.decode_attend_fv_workspace_bytes.restype = ctypes.c_size_t
lib.decode_attend_fv_workspace_bytes.argtypes = [_vp, _i32, _i32]
lib.decode_attend_fv.restype = ctypes.c_int
lib.decode_attend_fv.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp, _vp,
                                 ctypes.c_size_t, _vp]
lib.iskv_window_rows.restype = _i32
lib.iskv_window_rows.argtypes = [_i32, _i32, _i32]
lib.iskv_window_init.restype = ctypes.c_int
lib.iskv_window_init.argtypes = [ctypes.POINTER(_vp), _vp, _i32, _i32, _i32, _vp, _vp, _vp]
lib.iskv_window_protect.restype = ctypes.c_int
lib.iskv_window_protect.argtypes = [_vp, _vp, _pi32, _i32]
lib.iskv_window_append.restype = ctypes.c_int
lib.iskv_window_append.argtypes = [_vp, _vp, _i32, _i32, _pi32]
lib.iskv_window_append_batched.restype = ctypes.c_int
lib.iskv_window_append_batched.argtypes = [ctypes.POINTER(_vp), _i32, _vp, ctypes.c_int64, _i32, _i32, _pi32]
lib.iskv_window_exact.restype = ctypes.c_int
lib.iskv_window_exact.argtypes = [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _pi32]
lib.iskv_window_destroy.restype = None
lib.iskv_window_destroy.argtypes = [_vp]


class IskvError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {iskv_strerror(code)} ({code})")
        self.code = code


def iskv_strerror(code: int) -> str:
    return lib.iskv_strerror(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != 0:
        raise IskvError(code, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream_ptr(stream) -> int | None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


# ---- raw entry points (same names as the C ABI) ------------------------------
def isvd_workspace_bytes(cfg: IskvConfig) -> int:
    return int(lib.isvd_workspace_bytes(ctypes.byref(cfg)))


def isvd_init(cfg: IskvConfig, C, sigma, B, pos, workspace, stream=None) -> int:
    h = _vp()
    _check(lib.isvd_init(ctypes.byref(h), ctypes.byref(cfg), _ptr(C), _ptr(sigma), _ptr(B), _ptr(pos),
                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _stream_ptr(stream)), "isvd_init")
    return h.value


def isvd_merge_block(h: int, F, pos_F, b: int) -> None:
    _check(lib.isvd_merge_block(h, _ptr(F), _ptr(pos_F), int(b)), "isvd_merge_block")


def isvd_merge_block_batched(handles, F, F_stride: int, pos_F, pos_stride: int, b: int) -> None:
    arr = (_vp * len(handles))(*handles)
    _check(lib.isvd_merge_block_batched(arr, len(handles), _ptr(F), int(F_stride), _ptr(pos_F),
                                        int(pos_stride), int(b)), "isvd_merge_block_batched")


def isvd_reorth(h: int) -> None:
    _check(lib.isvd_reorth(h), "isvd_reorth")


def isvd_copy(dst: int, src: int) -> None:
    _check(lib.isvd_copy(dst, src), "isvd_copy")


def isvd_set_mode(h: int, mode: int) -> None:
    _check(lib.isvd_set_mode(h, int(mode)), "isvd_set_mode")


def isvd_refit_workspace_bytes(h: int) -> int:
    return int(lib.isvd_refit_workspace_bytes(h))


def isvd_refit(h: int, X, pos, n: int, iters: int, work) -> None:
    nbytes = 0 if work is None else work.numel() * work.element_size()
    _check(lib.isvd_refit(h, _ptr(X), _ptr(pos), int(n), int(iters), _ptr(work), nbytes), "isvd_refit")


def isvd_value_first_refit_workspace_bytes(h: int) -> int:
    return int(lib.isvd_value_first_refit_workspace_bytes(h))


def isvd_value_first_refit(h: int, F, pos_F, count: int, iters: int, work) -> None:
    nbytes = 0 if work is None else work.numel() * work.element_size()
    _check(lib.isvd_value_first_refit(h, _ptr(F), _ptr(pos_F), int(count), int(iters), _ptr(work), nbytes),
           "isvd_value_first_refit")


def iskv_prompt_split_workspace_bytes(L: int) -> int:
    return int(lib.iskv_prompt_split_workspace_bytes(int(L)))


def iskv_prompt_split(X, flags, L: int, D: int, mask: int, pos0: int, X_keep, pos_keep, X_rest, pos_rest, counts,
                      workspace, stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.iskv_prompt_split(_ptr(X), _ptr(flags), int(L), int(D), int(mask), int(pos0), _ptr(X_keep),
                                 _ptr(pos_keep), _ptr(X_rest), _ptr(pos_rest), _ptr(counts), _ptr(workspace),
                                 nbytes, _stream_ptr(stream)), "iskv_prompt_split")


def prompt_split(X, flags, mask: int, pos0: int = 0, stream=None):
    """Rows of X (fp32 [L, D] on the device) kept exact (flags & mask) and the
    others, each in position order with their positions; the two counts are
    read back. Returns (X_keep, pos_keep, X_rest, pos_rest) trimmed to them."""
    import torch
    L, D = int(X.shape[0]), int(X.shape[1])
    dev = X.device
    X_keep = torch.empty((max(L, 1), D), dtype=torch.float32, device=dev)
    X_rest = torch.empty((max(L, 1), D), dtype=torch.float32, device=dev)
    pos_keep = torch.empty((max(L, 1),), dtype=torch.int32, device=dev)
    pos_rest = torch.empty((max(L, 1),), dtype=torch.int32, device=dev)
    counts = torch.empty((2,), dtype=torch.int32, device=dev)
    ws = torch.empty((max(iskv_prompt_split_workspace_bytes(L), 1),), dtype=torch.uint8, device=dev)
    iskv_prompt_split(X, flags, L, D, mask, pos0, X_keep, pos_keep, X_rest, pos_rest, counts, ws, stream)
    nk, nr = (int(v) for v in counts.cpu().tolist())
    return X_keep[:nk], pos_keep[:nk], X_rest[:nr], pos_rest[:nr]


def prefill_init(kpath, vpath, K_pre, K_rot, V, Hkv: int, dh: int, block: int = 8, per_head: int = 128,
                 suffix_blocks: int = 4, v_radius: int = 32, v_window: int = 128, iters: int = 40):
    """Prompt initialisation (iS-KV notes §3.1, Algorithm 1) of one
    layer's key and value paths (fresh handles, fp32 rows on the device):
    exact sets from the post-RoPE keys K_rot (bf16 [L, Hkv * dh]), E_K = P_K
    and E_V = P_V | W_V; each path's other rows (pre-RoPE keys K_pre, values
    V) replaced by their fresh truncated SVD (isvd_refit) with positions
    saved. Returns ((K_exact, pos_K), (V_exact, pos_V), flags): the exact rows
    each path keeps, in position order, and the flags of every position."""
    import torch
    L = int(K_pre.shape[0])
    dev = K_pre.device
    flags = torch.empty((L,), dtype=torch.uint8, device=dev)
    ws = torch.empty((iskv_prompt_protect_workspace_bytes(L, Hkv, block, suffix_blocks),), dtype=torch.uint8,
                     device=dev)
    iskv_prompt_protect(K_rot, L, Hkv, dh, block, per_head, suffix_blocks, v_radius, v_window, flags, None, ws)
    out = []
    for path, X, mask in ((kpath, K_pre, 1), (vpath, V, 6)):
        Xk, pk, Xr, pr = prompt_split(X, flags, mask)
        if Xr.shape[0] > 0:
            path.refit(Xr, pr, iters=iters)
        out.append((Xk, pk))
    return out[0], out[1], flags


def iskv_prompt_protect_workspace_bytes(L: int, Hkv: int, block: int = 8, suffix_blocks: int = 4) -> int:
    return int(lib.iskv_prompt_protect_workspace_bytes(L, Hkv, block, suffix_blocks))


def iskv_prompt_protect(K_rot, L: int, Hkv: int, dh: int, block: int, per_head: int, suffix_blocks: int,
                        v_radius: int, v_window: int, flags, scores, workspace, stream=None) -> None:
    _check(lib.iskv_prompt_protect(_ptr(K_rot), int(L), int(Hkv), int(dh), int(block), int(per_head),
                                   int(suffix_blocks), int(v_radius), int(v_window), _ptr(flags), _ptr(scores),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream_ptr(stream)), "iskv_prompt_protect")


def prompt_protect(K_rot, Hkv: int, dh: int, block: int = 8, per_head: int = 128, suffix_blocks: int = 4,
                   v_radius: int = 32, v_window: int = 128, with_scores: bool = False, stream=None):
    """Exact-row masks (P_K, P_V, W_V) of a prompt from its post-RoPE keys
    (bf16 [L, Hkv * dh] on the device); optionally the block scores too."""
    import torch
    L = int(K_rot.shape[0])
    dev = K_rot.device
    flags = torch.empty((L,), dtype=torch.uint8, device=dev)
    nb = max(L // block - suffix_blocks, 0)
    scores = torch.empty((Hkv, nb), dtype=torch.float32, device=dev) if with_scores and nb > 0 else None
    ws = torch.empty((iskv_prompt_protect_workspace_bytes(L, Hkv, block, suffix_blocks),), dtype=torch.uint8,
                     device=dev)
    iskv_prompt_protect(K_rot, L, Hkv, dh, block, per_head, suffix_blocks, v_radius, v_window, flags, scores, ws,
                        stream)
    pk, pv, wv = (flags & 1) != 0, (flags & 2) != 0, (flags & 4) != 0
    return (pk, pv, wv, scores) if with_scores else (pk, pv, wv)


def isvd_query(h: int):
    n, k, st = _i32(), _i32(), _i32()
    _check(lib.isvd_query(h, ctypes.byref(n), ctypes.byref(k), ctypes.byref(st)), "isvd_query")
    return n.value, k.value, st.value


def isvd_query_state(h: int, count: int = 16):
    arr = (ctypes.c_int32 * count)()
    _check(lib.isvd_query_state(h, arr, count), "isvd_query_state")
    return list(arr)


def isvd_sym_eig(h: int, A, m: int, lam, V) -> None:
    _check(lib.isvd_sym_eig(h, _ptr(A), int(m), _ptr(lam), _ptr(V)), "isvd_sym_eig")


def isvd_set_timing(h: int, on: bool) -> None:
    _check(lib.isvd_set_timing(h, int(bool(on))), "isvd_set_timing")


MERGE_STAGES = ("project_residual", "residual_basis", "core_eig", "coord_update", "new_rows_basis")


def isvd_stage_times(h: int) -> dict:
    arr = (ctypes.c_float * len(MERGE_STAGES))()
    _check(lib.isvd_stage_times(h, arr, len(MERGE_STAGES)), "isvd_stage_times")
    return dict(zip(MERGE_STAGES, (float(x) for x in arr)))


def isvd_rows(h: int) -> int:
    return int(lib.isvd_rows(h))


def isvd_destroy(h: int) -> None:
    lib.isvd_destroy(h)


def kv_reconstruct(h: int, X_exact, pos_exact, n_exact: int, n_total: int, head_dim: int,
                   apply_rope: bool, rope_theta: float, out, out_dtype: int, stream=None) -> None:
    _check(lib.kv_reconstruct(h, _ptr(X_exact), _ptr(pos_exact), int(n_exact), int(n_total),
                              int(head_dim), int(bool(apply_rope)), float(rope_theta), _ptr(out),
                              int(out_dtype), _stream_ptr(stream)), "kv_reconstruct")


def kv_reconstruct_batched(handles, outs, n_totals, apply_rope, head_dim: int, rope_theta: float,
                           stream=None) -> None:
    """Compressed rows of several histories (bf16 outputs) in one launch."""
    k = len(handles)
    if not (len(outs) == len(n_totals) == len(apply_rope) == k):
        raise ValueError("kv_reconstruct_batched: one output, row count and RoPE flag per handle")
    hs = (_vp * k)(*handles)
    os_ = (_vp * k)(*[_ptr(o) for o in outs])
    nt = (ctypes.c_int32 * k)(*[int(x) for x in n_totals])
    rp = (ctypes.c_int32 * k)(*[int(bool(x)) for x in apply_rope])
    _check(lib.kv_reconstruct_batched(hs, k, os_, nt, rp, int(head_dim), float(rope_theta), _stream_ptr(stream)),
           "kv_reconstruct_batched")


def kv_scatter_exact(X_exact, pos_exact, n_exact: int, D: int, n_total: int, head_dim: int,
                     apply_rope: bool, rope_theta: float, out, out_dtype: int, stream=None) -> None:
    _check(lib.kv_scatter_exact(_ptr(X_exact), _ptr(pos_exact), int(n_exact), int(D), int(n_total),
                                int(head_dim), int(bool(apply_rope)), float(rope_theta), _ptr(out),
                                int(out_dtype), _stream_ptr(stream)), "kv_scatter_exact")


def decode_attend_workspace_bytes(batch: int, n: int, Hq: int, dh: int) -> int:
    return int(lib.decode_attend_workspace_bytes(batch, n, Hq, dh))


def decode_attend(q, K, V, batch: int, n: int, Hq: int, Hkv: int, dh: int, scale: float, out,
                  workspace, stream=None) -> None:
    _check(lib.decode_attend(_ptr(q), _ptr(K), _ptr(V), int(batch), int(n), int(Hq), int(Hkv),
                             int(dh), float(scale), _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "decode_attend")


def decode_attend_noalloc(q, K, V, batch: int, n: int, Hq: int, Hkv: int, dh: int, scale: float, out,
                          stream=None) -> None:
    """decode_attend with its partials in the library's fixed device scratch
    (no workspace, nothing allocated); see include/iskv.h for the size limit."""
    _check(lib.decode_attend_noalloc(_ptr(q), _ptr(K), _ptr(V), int(batch), int(n), int(Hq), int(Hkv), int(dh),
                                     float(scale), _ptr(out), _stream_ptr(stream)), "decode_attend_noalloc")


def decode_attend_fv_workspace_bytes(hv: int, n_exact: int, Hq: int) -> int:
    return int(lib.decode_attend_fv_workspace_bytes(hv, int(n_exact), int(Hq)))


def decode_attend_fv(q, K, hv: int, X_exact, pos_exact, n_exact: int, n_total: int, Hq: int, Hkv: int, dh: int,
                     scale: float, out, workspace, stream=None) -> None:
    _check(lib.decode_attend_fv(_ptr(q), _ptr(K), hv, _ptr(X_exact), _ptr(pos_exact), int(n_exact), int(n_total),
                                int(Hq), int(Hkv), int(dh), float(scale), _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream_ptr(stream)),
           "decode_attend_fv")


def iskv_window_rows(prot_cap: int, window: int, block: int) -> int:
    return int(lib.iskv_window_rows(prot_cap, window, block))


def iskv_window_init(h: int, prot_cap: int, window: int, block: int, rows, pos, stream=None) -> int:
    w = _vp()
    _check(lib.iskv_window_init(ctypes.byref(w), h, prot_cap, window, block, _ptr(rows), _ptr(pos),
                                _stream_ptr(stream)), "iskv_window_init")
    return w.value


def iskv_window_protect(w: int, rows, positions) -> None:
    arr = (ctypes.c_int32 * len(positions))(*[int(p) for p in positions])
    _check(lib.iskv_window_protect(w, _ptr(rows), arr, len(positions)), "iskv_window_protect")


def iskv_window_append(w: int, rows, pos0: int, count: int) -> int:
    m = _i32()
    _check(lib.iskv_window_append(w, _ptr(rows), int(pos0), int(count), ctypes.byref(m)),
           "iskv_window_append")
    return m.value


def iskv_window_append_batched(windows, rows, rows_stride: int, pos0: int, n: int) -> int:
    arr = (_vp * len(windows))(*windows)
    m = _i32()
    _check(lib.iskv_window_append_batched(arr, len(windows), _ptr(rows), int(rows_stride), int(pos0), int(n),
                                          ctypes.byref(m)), "iskv_window_append_batched")
    return m.value


def iskv_window_exact(w: int):
    r, p, c = _vp(), _vp(), _i32()
    _check(lib.iskv_window_exact(w, ctypes.byref(r), ctypes.byref(p), ctypes.byref(c)),
           "iskv_window_exact")
    return r.value, p.value, c.value


def iskv_window_destroy(w: int) -> None:
    lib.iskv_window_destroy(w)


# ---- owners of the device buffers behind one handle --------------------------
def _coord_dtype(torch, bf16: bool, fp16: bool):
    return torch.bfloat16 if bf16 else (torch.float16 if fp16 else torch.float32)


class IsvdPath:
    """One compressed (layer, K-or-V) path: torch tensors + the C handle."""

    def __init__(self, D: int, r_max: int, b_max: int, n_cap: int, reorth_every_rows: int = 0,
                 resid_rel_tol: float = 0.0, sync: bool = True, device="cuda", stream=None,
                 graphs: bool = True, _buffers=None, coords_bf16: bool = False, coords_fp16: bool = False):
        import torch
        if coords_bf16 and coords_fp16:
            raise ValueError("coords_bf16 and coords_fp16 are exclusive")
        flags = ((0 if sync else ISKV_NO_COORD_SYNC) | (0 if graphs else ISKV_NO_GRAPH) |
                 (ISKV_BF16_COORDS if coords_bf16 else 0) | (ISKV_FP16_COORDS if coords_fp16 else 0))
        self.cfg = IskvConfig(D, r_max, b_max, n_cap, reorth_every_rows, resid_rel_tol, flags)
        ws = isvd_workspace_bytes(self.cfg)
        if ws == 0:
            raise ValueError("invalid iskv configuration")
        if _buffers is not None:
            # carved by IsvdBatch from its shared allocation
            self.C, self.sigma, self.B, self.pos, self._ws_view = _buffers
            self.workspace = None
        else:
            dev = torch.device(device)
            # stored coordinates: fp32, or bf16 / fp16 (2-byte persistent factors)
            self.C = torch.empty((n_cap, r_max), dtype=_coord_dtype(torch, coords_bf16, coords_fp16), device=dev)
            self.sigma = torch.empty((r_max,), dtype=torch.float32, device=dev)
            self.B = torch.empty((D, r_max), dtype=torch.float32, device=dev)
            self.pos = torch.empty((n_cap,), dtype=torch.int32, device=dev)
            self.workspace = torch.empty((ws + 256,), dtype=torch.uint8, device=dev)
            off = (-self.workspace.data_ptr()) % 256
            self._ws_view = self.workspace[off:off + ws]
        self.stream = stream
        self.h = isvd_init(self.cfg, self.C, self.sigma, self.B, self.pos, self._ws_view, stream)

    def merge(self, F, pos_F) -> None:
        isvd_merge_block(self.h, F, pos_F, F.shape[0])

    def reorth(self) -> None:
        isvd_reorth(self.h)

    def refit(self, X, pos, iters: int = 40) -> None:
        """Fresh rank-r truncated SVD of the rows X (fp32 [n, D]) at positions pos."""
        import torch
        work = None
        if iters > 0:
            work = torch.empty((isvd_refit_workspace_bytes(self.h),), dtype=torch.uint8, device=self.C.device)
        isvd_refit(self.h, X, pos, int(X.shape[0]), iters, work)
        self._refit_work = work  # kept until the stream has used it

    def value_first_refit(self, F, pos_F, iters: int = 40) -> None:
        """The value first refit: fresh truncated SVD of [history; F]."""
        import torch
        work = torch.empty((isvd_value_first_refit_workspace_bytes(self.h),), dtype=torch.uint8,
                           device=self.C.device)
        isvd_value_first_refit(self.h, F, pos_F, int(F.shape[0]), iters, work)
        self._refit_work = work  # kept until the stream has used it

    def copy_from(self, other: "IsvdPath") -> None:
        """Replace this path's history by a copy of other's (isvd_copy)."""
        isvd_copy(self.h, other.h)

    def set_mode(self, mode: int) -> None:
        """0 (full merge), ISKV_NO_COORD_SYNC (basis-only) or ISKV_FROZEN_BASIS."""
        isvd_set_mode(self.h, mode)

    def query(self):
        return isvd_query(self.h)

    def state(self):
        return isvd_query_state(self.h)

    def set_timing(self, on: bool) -> None:
        isvd_set_timing(self.h, on)

    def stage_times(self) -> dict:
        return isvd_stage_times(self.h)

    def sym_eig(self, A):
        """Eigenpairs of a symmetric fp64 device matrix with the core eigensolver."""
        import torch
        m = A.shape[0]
        lam = torch.empty((m,), dtype=torch.float64, device=A.device)
        V = torch.empty((m, m), dtype=torch.float64, device=A.device)
        isvd_sym_eig(self.h, A.contiguous(), m, lam, V)
        return lam, V

    @property
    def n(self) -> int:
        return isvd_rows(self.h)

    def reconstruct(self, out, n_total: int, X_exact=None, pos_exact=None, head_dim: int = 128,
                    rope: bool = False, theta: float = 500000.0, stream=None) -> None:
        import torch
        dt = ISKV_OUT_BF16 if out.dtype == torch.bfloat16 else ISKV_OUT_FP32
        n_exact = 0 if X_exact is None else int(X_exact.shape[0])
        kv_reconstruct(self.h, X_exact, pos_exact, n_exact, n_total, head_dim, rope, theta, out, dt,
                       stream if stream is not None else self.stream)

    def close(self) -> None:
        if getattr(self, "h", None):
            isvd_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _round256(x: int) -> int:
    return (x + 255) // 256 * 256


class IsvdBatch:
    """`count` paths with one configuration carved from one allocation at a
    fixed per-path stride, so that one isvd_merge_block_batched call merges a
    block into every path (iS-KV notes §2.2: each (sequence, layer, K/V) path
    is compressed independently). ``paths[z]`` is an ordinary IsvdPath (its
    C, sigma, B, pos and workspace are views into the shared allocation) and
    can be merged, reconstructed and queried on its own as well."""

    def __init__(self, count: int, D: int, r_max: int, b_max: int, n_cap: int, reorth_every_rows: int = 0,
                 resid_rel_tol: float = 0.0, sync: bool = True, device="cuda", stream=None,
                 graphs: bool = True, window: int | None = None, block: int | None = None, prot_cap: int = 0,
                 coords_bf16: bool = False, coords_fp16: bool = False):
        import torch
        if count < 1:
            raise ValueError("count must be >= 1")
        cfg = IskvConfig(D, r_max, b_max, n_cap, reorth_every_rows, resid_rel_tol, 0)
        ws = isvd_workspace_bytes(cfg)
        if ws == 0:
            raise ValueError("invalid iskv configuration")
        csz = 2 if (coords_bf16 or coords_fp16) else 4
        sizes = [n_cap * r_max * csz, r_max * 4, D * r_max * 4, n_cap * 4, ws]
        wrows = 0
        if window is not None:  # exact window + pending FIFO of every path in the same slot
            wrows = iskv_window_rows(prot_cap, window, block if block is not None else b_max)
            sizes += [wrows * D * 4, wrows * 4]
        offs = []
        o = 0
        for nb in sizes:
            offs.append(o)
            o += _round256(nb)
        self.stride = o  # bytes from one path's buffers to the next one's
        self.count = count
        self.D, self.b_max = D, b_max
        self.stream = stream
        self.blob = torch.empty((count * self.stride + 256,), dtype=torch.uint8, device=torch.device(device))
        base = (-self.blob.data_ptr()) % 256
        self.paths = []
        self.windows = []
        for z in range(count):
            z0 = base + z * self.stride

            def view(i, dtype, shape):
                return self.blob[z0 + offs[i]:z0 + offs[i] + sizes[i]].view(dtype).view(shape)

            bufs = (view(0, _coord_dtype(torch, coords_bf16, coords_fp16), (n_cap, r_max)),
                    view(1, torch.float32, (r_max,)),
                    view(2, torch.float32, (D, r_max)), view(3, torch.int32, (n_cap,)),
                    self.blob[z0 + offs[4]:z0 + offs[4] + ws])
            self.paths.append(IsvdPath(D, r_max, b_max, n_cap, reorth_every_rows, resid_rel_tol, sync,
                                       device, stream, graphs, _buffers=bufs, coords_bf16=coords_bf16,
                                       coords_fp16=coords_fp16))
            if wrows:
                self.windows.append(ExactWindow(self.paths[-1], window, block if block is not None else b_max,
                                                prot_cap, stream,
                                                _buffers=(view(5, torch.float32, (wrows, D)),
                                                          view(6, torch.int32, (wrows,)))))
        self.handles = [p.h for p in self.paths]

    def merge(self, F, pos_F) -> None:
        """F: [count, b, D] fp32, pos_F: [count, b] int32 (contiguous in the
        last two dimensions); block z goes to path z."""
        if F.dim() != 3 or F.shape[0] != self.count or F.shape[2] != self.D:
            raise ValueError("F must be [count, b, D]")
        if F.stride(2) != 1 or F.stride(1) != self.D or pos_F.stride(-1) != 1:
            raise ValueError("F rows and pos_F must be contiguous")
        b = F.shape[1]
        isvd_merge_block_batched(self.handles, F, F.stride(0), pos_F, pos_F.stride(0), b)

    def append(self, rows, pos0: int) -> int:
        """Append rows[z] (rows: [count, n, D] fp32, rows contiguous) to the
        exact window of path z at positions pos0.., merging every full block
        of all paths in one batched launch sequence; returns the merges made."""
        if not self.windows:
            raise ValueError("IsvdBatch was created without windows")
        if rows.dim() != 3 or rows.shape[0] != self.count or rows.shape[2] != self.D:
            raise ValueError("rows must be [count, n, D]")
        if rows.stride(2) != 1 or rows.stride(1) != self.D:
            raise ValueError("rows must be contiguous within each path")
        return iskv_window_append_batched([w.w for w in self.windows], rows, rows.stride(0), pos0, rows.shape[1])

    def __len__(self) -> int:
        return self.count

    def __getitem__(self, z: int) -> IsvdPath:
        return self.paths[z]

    def close(self) -> None:
        for w in getattr(self, "windows", []):
            w.close()
        for p in getattr(self, "paths", []):
            p.close()


class ExactWindow:
    """Exact recent window + pending FIFO feeding one IsvdPath (iS-KV notes §3.2)."""

    def __init__(self, path: IsvdPath, window: int, block: int, prot_cap: int = 0, stream=None,
                 _buffers=None):
        import torch
        self.path = path
        rows = iskv_window_rows(prot_cap, window, block)
        dev = path.C.device
        if _buffers is not None:  # carved by IsvdBatch from its shared allocation
            self.rows, self.pos = _buffers
        else:
            self.rows = torch.empty((rows, path.cfg.D), dtype=torch.float32, device=dev)
            self.pos = torch.empty((rows,), dtype=torch.int32, device=dev)
        self.w = iskv_window_init(path.h, prot_cap, window, block, self.rows, self.pos,
                                  stream if stream is not None else path.stream)

    def protect(self, rows, positions) -> None:
        iskv_window_protect(self.w, rows, positions)

    def append(self, rows, pos0: int) -> int:
        return iskv_window_append(self.w, rows, pos0, rows.shape[0])

    def close(self) -> None:
        if getattr(self, "w", None):
            iskv_window_destroy(self.w)
            self.w = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
