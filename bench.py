#!/usr/bin/env python3
"""Benchmark of the iS-KV hot path on one MI355X.

Workload: the Llama-8B-shaped stream, D = 8 KV heads x 128 = 1024, rank
budget r = 256, block b = 32, exact recent window w = 128, with a key path
(sigma_i = exp(-i/40) + 0.01) and a value path of the same shape
(sigma_i = (1+i)^-1/2). Both paths are first filled with 16,384 rows; then one
timed step is one pass of the whole hot path at n ~ 16K:
  * ingest b new K rows and b new V rows through the exact window; the rows
    leaving the window become a pending block that is merged (one iSVD merge
    per path; re-orthogonalisation every 256 folded rows). The K and V paths
    are two handles on two HIP streams, so their merges overlap;
    `--batched-kv` instead carves them from one allocation and runs both merges
    as one batched launch sequence (iskv_window_append_batched);
  * reconstruct the dense K cache (bf16, RoPE theta = 500000 at every
    position) and V cache (bf16) from the factors plus the exact window;
  * GQA decode attention of one query (32 heads over 8 KV heads, d_h = 128)
    over the reconstructed cache.
The headline value is iSVD merges per second (two per step). Inputs are
synthetic and resident in HBM before the timed region.

Prints ONE JSON line (rank 0). `--gpus N` with N > 1 exits: the benchmark runs on
one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D, R, BLK, WIN, N0 = 1024, 256, 32, 128, 16384
HQ, HKV, DH, THETA = 32, 8, 128, 500000.0
HBM_PEAK_GBPS = 8000.0
CALIB_BYTES = 256 << 20
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
TIMED_MERGES = 8  # merges run once more with stage events after the timed region
MODE_MERGES = 16  # merges timed in each merge mode at the end of the run
SINGLE_REPS = 20  # one-path reconstruction launches timed after the timed region


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--batch-paths", type=int, default=1024,
                    help="paths of the batch leg (16 sequences x 32 layers x K/V; 0 skips it)")
    ap.add_argument("--batch-rows", type=int, default=32768, help="rows per path before the batch leg's timing")
    ap.add_argument("--batch-steps", type=int, default=16, help="timed batched merges of the batch leg")
    ap.add_argument("--batched-kv", action="store_true",
                    help="K and V carved from one allocation, merged as one batched launch sequence")
    ap.add_argument("--main-only", action="store_true",
                    help="only the timed K/V steps and their stage breakdown (for counter passes)")
    ap.add_argument("--prompt-decode-only", action="store_true",
                    help="only the 64K-row r = 512 prompt + decode leg, printed as its own JSON object "
                         "(for kernel traces of the high-rank merge and the block Jacobi)")
    ap.add_argument("--no-graphs", action="store_true",
                    help="enqueue every kernel directly instead of replaying recorded HIP graphs "
                         "(same kernels; for kernel-trace profilers)")
    return ap.parse_args()


def profiled_traffic(name):
    """HBM bytes per dispatch from a committed rocprofv3 counter summary under
    profiles/, or None when the kernel source changed since it was measured."""
    import hashlib
    import re
    prof = os.path.join(ROOT, "profiles", name)
    try:
        text = open(prof).read()
        d = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        src = open(os.path.join(ROOT, d["source"]), "rb").read()
    except (OSError, AttributeError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != d["source_sha256"]:
        return None
    return float(d["traffic_bytes_per_dispatch"])


def prefill_leg(args, K, torch, dev):
    """Prompt initialisation of one layer at the 64K-stream shape's prompt:
    L = 8192 rows, D = 1024 (8 KV heads x 128), r_K = 192 and r_V = 320
    (the K and V stream ranks), b = 64; anomaly scores on synthetic post-RoPE keys with 12 kept blocks per
    head (about 10% of the blocks, plus the value neighbourhoods), each path's
    non-exact rows refit (the fresh truncated SVD: 24 subspace iterations on
    the key path, 40 on the value path), then the value first refit with the
    next 320 rows. Each stage timed on the null stream; median
    of 2 runs after one warm-up."""
    import synth
    # subspace iterations of the refits: the key spectrum converges in about
    # 15 (24 kept), the value spectrum's flatter tail needs about 40
    L, hkv, dh, r_k, r, per_head, iters_k, iters = 8192, 8, 128, 192, 320, 12, 24, 40
    Kb = torch.from_numpy(synth.prompt_keys(L, hkv, dh, 41)).to(dev).bfloat16()
    K_pre = torch.from_numpy(synth.kv_stream(synth.StreamSpec(D, L, "exp40+0.01", 0.0, 40))).to(dev)
    Vall = torch.from_numpy(synth.kv_stream(synth.StreamSpec(D, L + r, "invsqrt", 0.0, 41))).to(dev)
    V, Vnew = Vall[:L], Vall[L:]
    pos_new = torch.arange(L, L + r, dtype=torch.int32, device=dev)
    flags = torch.empty((L,), dtype=torch.uint8, device=dev)
    ws = torch.empty((K.iskv_prompt_protect_workspace_bytes(L, hkv),), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        torch.cuda.synchronize()
        ev[0].record()
        out = fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]), out

    runs, rows = [], {}
    for rep in range(3):
        kp = K.IsvdPath(D=D, r_max=r_k, b_max=64, n_cap=L + r, device=dev)
        vp = K.IsvdPath(D=D, r_max=r, b_max=64, n_cap=L + r, device=dev)
        t = {}
        t["protect_ms"], _ = timed(lambda: K.iskv_prompt_protect(Kb, L, hkv, dh, 8, per_head, 4, 32, 128, flags,
                                                                  None, ws))
        t["split_ms"], (sk, sv) = timed(lambda: (K.prompt_split(K_pre, flags, 1), K.prompt_split(V, flags, 6)))
        t["refit_k_ms"], _ = timed(lambda: kp.refit(sk[2], sk[3], iters=iters_k))
        t["refit_v_ms"], _ = timed(lambda: vp.refit(sv[2], sv[3], iters=iters))
        t["value_first_refit_ms"], _ = timed(lambda: vp.value_first_refit(Vnew, pos_new, iters=iters))
        rows = {"exact_k": int(sk[0].shape[0]), "refit_k": int(sk[2].shape[0]), "exact_v": int(sv[0].shape[0]),
                "refit_v": int(sv[2].shape[0]), "value_first_refit": int(sv[2].shape[0]) + r}
        if rep > 0:
            runs.append(t)
        kp.close()
        vp.close()
    res = {k: float(np.median([u[k] for u in runs])) for k in runs[0]}
    res.update({"rows": rows, "L": L, "D": D, "r_k": r_k, "r_v": r, "b": 64, "iters_k": iters_k, "iters_v": iters,
                "per_head": per_head})
    return res


def prompt_decode_leg(args, K, torch, dev):
    """The 64K-row prompt + decode stream at its full size: D = 1024, r = 512,
    b = 64, key spectrum, rows drawn on the device. The factor of its first
    65,536 - 18 x 64 rows comes from the fresh truncated SVD (isvd_refit:
    the prompt's factor step of Algorithm 1, here over every row), then 16
    merges are timed at n ~ 64K (re-orthogonalisation every 256 rows,
    recorded sequences, HIP events on the path's stream). The workload
    reconstructs all rows every 64 decode steps: that reconstruction (bf16 +
    RoPE, all n rows) is timed 10 times, with its bytes, MFMA fraction and
    cost per decode step (one 64th)."""
    import synth
    r, b, N, merges = 512, 64, 65536, 16
    n0 = N - (merges + 2) * b
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        X = synth.DeviceStreams(1, 1, D, 64, dev).rows(N)[0].contiguous()
        pos = torch.arange(N, dtype=torch.int32, device=dev)
    st.synchronize()
    p = K.IsvdPath(D=D, r_max=r, b_max=b, n_cap=N, reorth_every_rows=256, device=dev, stream=st,
                   graphs=not args.no_graphs)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(st)
    p.refit(X[:n0], pos[:n0])
    ev[1].record(st)
    st.synchronize()
    refit_ms = ev[0].elapsed_time(ev[1])
    for j in range(2):  # warm-up (records the sequences)
        s0 = n0 + j * b
        p.merge(X[s0:s0 + b], pos[s0:s0 + b])
    st.synchronize()
    ev[0].record(st)
    for j in range(2, merges + 2):
        s0 = n0 + j * b
        p.merge(X[s0:s0 + b], pos[s0:s0 + b])
    ev[1].record(st)
    st.synchronize()
    merge_ms = ev[0].elapsed_time(ev[1]) / merges
    n, k, status = p.query()
    state = p.state()
    out = torch.empty((N, D), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        p.reconstruct(out, N, head_dim=DH, rope=True, theta=THETA, stream=st)
    ev[0].record(st)
    reps = 10
    for _ in range(reps):
        p.reconstruct(out, N, head_dim=DH, rope=True, theta=THETA, stream=st)
    ev[1].record(st)
    st.synchronize()
    rec_ms = ev[0].elapsed_time(ev[1]) / reps
    rec_bytes = n * r * 4 + r * D * 2 + n * D * 2
    rec_flops = 2.0 * n * r * D
    p.close()
    return {"rows": n, "rank": k, "r": r, "b": b, "status": status, "refit_rows": n0, "refit_ms": refit_ms,
            "merge_ms": merge_ms, "merges": merges,
            "last_core_solve": {"flags": state[11], "steps": state[12], "sweeps": state[7]},
            "reconstruct_ms": rec_ms, "reconstruct_bytes": rec_bytes,
            "reconstruct_GBps": rec_bytes / (rec_ms * 1e-3) / 1e9,
            "reconstruct_hbm_frac": rec_bytes / (rec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "reconstruct_mfma_frac": rec_flops / (rec_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "reconstruct_ms_per_step": rec_ms / 64,
            "what": "64K-row key stream at r=512, b=64 (core 576): factor of the first rows by the fresh "
                    "truncated SVD, merges timed at n~64K, full reconstruction every 64 steps"}


def batch_leg(args, K, torch, dev):
    """The batch workload: 16 sequences x 32 layers x {K, V} = 1024
    independent paths of 32,768 rows (D = 1024, r = 256, b = 32), carved from
    one allocation. A key-spectrum and a value-spectrum path are factored
    from 32,768 rows each (isvd_refit, the fresh truncated SVD), every path
    of the batch starts as a copy of the one of its kind (isvd_copy), and
    from then on each path takes its own rows (synth.DeviceStreams, one draw
    per path per block). Timed: --batch-steps batched merges, one b-row block
    per path each (isvd_merge_block_batched, re-orthogonalisation every 256
    rows), then two more with stage events."""
    import synth
    P, n0, steps = args.batch_paths, args.batch_rows, args.batch_steps
    warm = 2
    st = torch.cuda.Stream()
    n_cap = n0 + (steps + warm + 2) * BLK
    with torch.cuda.stream(st):
        ds = synth.DeviceStreams(P, P // 2, D, 1000, dev)
        bat = K.IsvdBatch(P, D=D, r_max=R, b_max=BLK, n_cap=n_cap, reorth_every_rows=256, device=dev, stream=st,
                          graphs=not args.no_graphs)
        t0 = time.perf_counter()
        seeds = []
        for kind, spec in ((0, "exp40+0.01"), (1, "invsqrt")):
            Xs = torch.from_numpy(synth.kv_stream(synth.StreamSpec(D, n0, spec, 0.0, 1000 + kind))).to(dev)
            ps = torch.arange(n0, dtype=torch.int32, device=dev)
            src = K.IsvdPath(D=D, r_max=R, b_max=BLK, n_cap=n0, reorth_every_rows=256, device=dev, stream=st,
                             graphs=False)
            src.refit(Xs, ps, iters=24 if kind == 0 else 40)
            seeds.append(src)
        st.synchronize()
        for z in range(P):
            bat.paths[z].copy_from(seeds[0 if z < P // 2 else 1])
        st.synchronize()
        init_s = time.perf_counter() - t0
        for sp in seeds:
            sp.close()
        cursor = n0
        pos = torch.empty((P, BLK), dtype=torch.int32, device=dev)

        def one_step():
            nonlocal cursor
            rows = ds.rows(BLK).contiguous()
            pos.copy_(torch.arange(cursor, cursor + BLK, dtype=torch.int32, device=dev).expand(P, BLK))
            bat.merge(rows, pos)
            cursor += BLK

        for _ in range(warm):
            one_step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.synchronize()
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(steps):
            one_step()
        e1.record(st)
        st.synchronize()
        wall = time.perf_counter() - t0
        bat.paths[0].set_timing(True)
        stage = []
        for _ in range(2):
            one_step()
            stage.append(bat.paths[0].stage_times())
        bat.paths[0].set_timing(False)
        st.synchronize()
        # the decode step over the compressed caches: per sequence, its L
        # layers' K and V histories rebuilt by kv_reconstruct_batched launches
        # of 16 layers each (32 paths, RoPE on the keys), then one
        # decode_attend over the L layers as a batch (32 query heads, 8 KV
        # heads); every sequence in turn, timed with HIP events
        dec = None
        L = min(32, P // 2)  # layers per sequence (32: 16 sequences x 32 layers at P = 1024)
        nseq = (P // 2) // L if L > 0 else 0
        LC = 16  # layers per reconstruction launch (2 LC <= 32 paths)
        if nseq > 0:
            n_dec = bat.paths[0].n
            Kall = torch.empty((L, n_dec, D), dtype=torch.bfloat16, device=dev)
            Vall = torch.empty((L, n_dec, D), dtype=torch.bfloat16, device=dev)
            qd = torch.from_numpy(np.random.default_rng(9).standard_normal((L, HQ, DH)).astype(np.float32)).to(
                dev).bfloat16()
            od = torch.empty((L, HQ, DH), dtype=torch.bfloat16, device=dev)
            wsd = torch.empty(K.decode_attend_workspace_bytes(L, n_dec, HQ, DH), dtype=torch.uint8, device=dev)
            ed = [torch.cuda.Event(enable_timing=True) for _ in range(3 * nseq)]
            nlaunch = (L + LC - 1) // LC

            def decode(sq, evs):
                if evs:
                    evs[0].record(st)
                for l0 in range(0, L, LC):
                    ls = range(l0, min(L, l0 + LC))
                    hs = [bat.paths[sq * L + l].h for l in ls] + [bat.paths[P // 2 + sq * L + l].h for l in ls]
                    K.kv_reconstruct_batched(hs, [Kall[l] for l in ls] + [Vall[l] for l in ls],
                                             [n_dec] * (2 * len(ls)), [True] * len(ls) + [False] * len(ls), DH,
                                             THETA, stream=st)
                if evs:
                    evs[1].record(st)
                K.decode_attend(qd, Kall, Vall, L, n_dec, HQ, HKV, DH, DH ** -0.5, od, wsd, stream=st)
                if evs:
                    evs[2].record(st)

            decode(0, None)
            st.synchronize()
            for sq in range(nseq):
                decode(sq, ed[3 * sq:3 * sq + 3])
            st.synchronize()
            rec_ms = float(np.mean([ed[3 * i].elapsed_time(ed[3 * i + 1]) for i in range(nseq)])) / nlaunch
            att_ms = float(np.mean([ed[3 * i + 1].elapsed_time(ed[3 * i + 2]) for i in range(nseq)]))
            rec_bytes = 2 * LC * (n_dec * R * 4 + R * D * 2 + n_dec * D * 2)
            att_bytes = 2 * L * n_dec * D * 2
            dec = {"sequences": nseq, "layers": L, "rows": n_dec,
                   "reconstruct_ms_per_launch": rec_ms, "paths_per_launch": 2 * LC,
                   "reconstruct_launches_per_sequence": nlaunch,
                   "reconstruct_algorithmic_bytes_per_launch": rec_bytes,
                   "reconstruct_GBps": rec_bytes / (rec_ms * 1e-3) / 1e9,
                   "reconstruct_hbm_frac": rec_bytes / (rec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                   "reconstruct_mfma_frac": 2 * LC * 2.0 * n_dec * R * D / (rec_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                   "attend_ms_per_launch": att_ms, "attend_batch": L,
                   "attend_GBps": att_bytes / (att_ms * 1e-3) / 1e9,
                   "decode_ms_all_sequences": nseq * (nlaunch * rec_ms + att_ms),
                   "what": f"per sequence: kv_reconstruct_batched over its {L} layers' K (RoPE) and V paths, "
                           f"{2 * LC} paths per launch, then one decode_attend over the {L} layers (batch {L}, "
                           f"32 q / 8 kv heads, bf16)"}
            del Kall, Vall, wsd
    ms = e0.elapsed_time(e1)
    states = [p.state() for p in bat.paths[:: max(1, P // 4)]]
    n_end = bat.paths[0].n
    bat.close()
    stage_ms = {k: float(np.mean([r[k] for r in stage])) for k in stage[0]}
    cu_bytes = P * 2.0 * (n_end - BLK) * R * 4
    return {"paths": P, "rows_per_path": n0, "block": BLK, "rank": R, "steps": steps,
            "merges_per_s": P * steps / wall, "ms_per_batched_merge": ms / steps,
            "merges_per_s_events": P * steps / (ms * 1e-3), "init_s": init_s,
            "stage_ms_per_batched_merge": stage_ms,
            "coord_update_GBps": cu_bytes / (stage_ms["coord_update"] * 1e-3) / 1e9,
            "core_solver_flags_sampled": [c[11] for c in states], "rows_at_end": n_end,
            "decode_step": dec,
            "workload": f"{P} independent paths ({P // 2} K, {P // 2} V spectra: 16 sequences x 32 layers x K/V "
                        f"when P = 1024), n={n0}, D={D}, r={R}, b={BLK}, reorth every 256 rows; paths start as "
                        f"copies of a K and a V factor of {n0} rows (fresh truncated SVD) and take their own "
                        f"rows, drawn on the device"}


def coords_leg(args, K, torch, dev, Xk, Kc):
    """fp32 against 2-byte (bf16, fp16) stored coordinates on three fresh K
    paths of N0 rows each, filled by merges and then timed the same way:
    MODE_MERGES merges (with re-orthogonalisation every 256 rows), 10
    reconstructions (bf16 with RoPE) and 10 factor-aware attentions (all rows
    compressed). After the fill, each path's factor drift of eq.(14) (relative
    error of C B^T against the N0 rows, minus that of their fresh rank-R
    truncated SVD; the latter from the eigenvalues of X^T X in float64) and
    its device status word (fp16 overflow guard) are recorded."""
    st = torch.cuda.Stream()
    n_fill, extra = N0, (MODE_MERGES + 2) * BLK
    Xd = torch.from_numpy(Xk[:n_fill + extra]).to(dev)
    pos = torch.arange(n_fill + extra, dtype=torch.int32, device=dev)
    rng = np.random.default_rng(6)
    q = torch.from_numpy(rng.standard_normal((HQ, DH)).astype(np.float32)).to(dev).bfloat16()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    # the fresh truncated SVD's error of the filled rows: sum of the trailing
    # eigenvalues of X^T X
    X64 = Xd[:n_fill].double()
    lam = torch.linalg.eigvalsh(X64.T @ X64).flip(0).clamp_min(0)
    nx = float(torch.sqrt(lam.sum()))
    fresh_rel = float(torch.sqrt(lam[R:].sum())) / nx
    res, outs = {}, {}
    for fmt in ("fp32", "bf16", "fp16"):
        p = K.IsvdPath(D=D, r_max=R, b_max=BLK, n_cap=n_fill + extra, reorth_every_rows=256, device=dev,
                       stream=st, graphs=not args.no_graphs, coords_bf16=fmt == "bf16", coords_fp16=fmt == "fp16")
        for s0 in range(0, n_fill, BLK):
            p.merge(Xd[s0:s0 + BLK], pos[s0:s0 + BLK])
        st.synchronize()
        n = p.n
        nq, kq, status = p.query()
        inc = p.C[:n, :kq].double() @ p.B[:, :kq].double().T  # rows in position order (pos = 0 .. n-1)
        inc_rel = float(torch.linalg.norm(X64 - inc)) / nx
        del inc
        out = torch.empty((n, D), dtype=torch.bfloat16, device=dev)
        of = torch.empty((HQ, DH), dtype=torch.bfloat16, device=dev)
        wsf = torch.empty(K.decode_attend_fv_workspace_bytes(p.h, 0, HQ), dtype=torch.uint8, device=dev)

        def timed(fn, reps):
            for _ in range(2):
                fn()
            ev[0].record(st)
            for _ in range(reps):
                fn()
            ev[1].record(st)
            st.synchronize()
            return ev[0].elapsed_time(ev[1]) / reps

        r_ms = timed(lambda: p.reconstruct(out, n, head_dim=DH, rope=True, theta=THETA, stream=st), 10)
        f_ms = timed(lambda: K.decode_attend_fv(q, Kc, p.h, None, None, 0, n, HQ, HKV, DH, DH ** -0.5, of, wsf,
                                                stream=st), 10)
        outs[fmt] = (out.float(), of.float())
        cur = [n_fill]

        def one_merge():
            s0 = cur[0]
            p.merge(Xd[s0:s0 + BLK], pos[s0:s0 + BLK])
            cur[0] += BLK

        m_ms = timed(one_merge, MODE_MERGES)
        res[fmt] = {"merge_ms": m_ms, "recon_ms": r_ms, "factor_v_ms": f_ms,
                    "coordinate_bytes": n * R * (4 if fmt == "fp32" else 2),
                    "drift_eq14": inc_rel - fresh_rel, "status": int(status)}
        p.close()
    del X64
    res["rows"] = n_fill
    res["fresh_svd_rel_err"] = fresh_rel
    ra, fa = outs["fp32"]
    for fmt in ("bf16", "fp16"):
        rb, fb = outs[fmt]
        res[fmt]["drift_minus_fp32"] = res[fmt]["drift_eq14"] - res["fp32"]["drift_eq14"]
        res[fmt]["recon_rel_diff"] = float(torch.linalg.norm(rb - ra) / torch.linalg.norm(ra))
        res[fmt]["factor_v_max_abs_diff"] = float((fb - fa).abs().max())
    return res


def cpu_baseline(Xk, Xv, seconds):
    """The oracle (float64 NumPy/LAPACK) timed on the host on a bounded sample,
    with the BLAS on all the host's threads and again on one thread.

    Sample: both paths start from a factorisation of their first 16,384 rows
    (the oracle's fresh truncated SVD, not timed); then whole steps (merge K,
    merge V, reconstruct K with RoPE and V, attention) are timed until
    `seconds` elapse (half of that on one thread). Reported in merges/s like
    the GPU value.
    """
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    res = _cpu_steps(Xk, Xv, seconds)
    res["cores"] = int(threads)
    with threadpool_limits(limits=1):
        one = _cpu_steps(Xk, Xv, seconds / 2)
    one["cores"] = 1
    res["one_thread"] = one
    res["host"] = {"sched_getaffinity": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
                   "blas": sorted({p.get("internal_api", "?") for p in threadpool_info()})}
    return res


def _cpu_steps(Xk, Xv, seconds):
    import oracle as O
    facs = []
    for X in (Xk, Xv):
        u, s, vt = np.linalg.svd(X[:N0].astype(np.float64), full_matrices=False)
        facs.append(O.Factor(U=u[:, :R], sigma=s[:R], B=vt[:R].T.copy(), pos=np.arange(N0)))
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, HQ, DH))
    steps, merges = 0, 0
    t0 = time.perf_counter()
    while True:
        s0 = N0 + steps * BLK
        for i, X in enumerate((Xk, Xv)):
            facs[i] = O.merge(facs[i], X[s0:s0 + BLK], np.arange(s0, s0 + BLK), R)
            merges += 1
        n = facs[0].n
        Kc = O.reconstruct(facs[0], np.zeros((0, D)), [], n, DH, True, THETA)
        Vc = O.reconstruct(facs[1], np.zeros((0, D)), [], n, DH, False)
        O.attend(q, Kc.reshape(1, n, HKV, DH), Vc.reshape(1, n, HKV, DH), DH ** -0.5)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds or s0 + 2 * BLK > Xk.shape[0]:
            break
    return {"value": merges / el, "unit": "merges/s", "kind": "oracle",
            "sample": f"{steps} whole steps (2 merges at n={N0}..{N0 + steps * BLK}, K+V reconstruction "
                      f"incl. RoPE, attention) from a fresh factorisation of 16,384 rows, float64, "
                      f"{el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path "
              "(every (sequence, layer, K/V) stream is independent of the others).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import online_rank_kv_amd as K

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.prompt_decode_only:
        print(json.dumps({"prompt_decode_64k": prompt_decode_leg(args, K, torch, dev)}), flush=True)
        return
    steps, warm = args.steps, args.warmup
    n_rows = N0 + (steps + warm + 4 + TIMED_MERGES + 3 * (MODE_MERGES + 2)) * BLK + WIN
    t_gen = time.perf_counter()
    Xk = synth.kv_stream(synth.StreamSpec(D, n_rows, "exp40+0.01", 0.0, 0))
    Xv = synth.kv_stream(synth.StreamSpec(D, n_rows, "invsqrt", 0.0, 1))
    gen_s = time.perf_counter() - t_gen

    batched = args.batched_kv
    if batched:
        # K and V carved from one allocation: every merge / window kernel runs
        # once over both paths (grid z = path) on one stream
        st = torch.cuda.Stream()
        streams = [st, torch.cuda.Stream()]  # the second only runs the V reconstruction
        with torch.cuda.stream(st):
            bat = K.IsvdBatch(2, D=D, r_max=R, b_max=BLK, n_cap=n_rows, reorth_every_rows=256, device=dev,
                              stream=st, graphs=not args.no_graphs, window=WIN, block=BLK)
            Xs = torch.from_numpy(np.stack([Xk, Xv])).to(dev)  # [2, n_rows, D]
            st.synchronize()
        paths, wins = bat.paths, bat.windows
        Xd = [Xs[0], Xs[1]]

        def ingest(s0, e0):
            bat.append(Xs[:, s0:e0], s0)
    else:
        # one HIP stream per path: the K and V merges (and their reconstructions)
        # are independent chains of small launches and run concurrently
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        paths, wins, Xd = [], [], []
        for X, st in zip((Xk, Xv), streams):
            with torch.cuda.stream(st):
                p = K.IsvdPath(D=D, r_max=R, b_max=BLK, n_cap=n_rows, reorth_every_rows=256, device=dev,
                               stream=st, graphs=not args.no_graphs)
                paths.append(p)
                wins.append(K.ExactWindow(p, window=WIN, block=BLK, stream=st))
                Xd.append(torch.from_numpy(X).to(dev))
                st.synchronize()

        def ingest(s0, e0):
            for i in range(2):
                wins[i].append(Xd[i][s0:e0], s0)
    # fill both paths with the first N0 rows (+ window)
    t_fill = time.perf_counter()
    for s in range(0, N0 + WIN, 512):
        ingest(s, min(s + 512, N0 + WIN))
    for st in streams:
        st.synchronize()
    fill_s = time.perf_counter() - t_fill
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.standard_normal((1, HQ, DH)).astype(np.float32)).to(dev).bfloat16()
    o = torch.empty((1, HQ, DH), dtype=torch.bfloat16, device=dev)
    Kc = torch.empty((n_rows, D), dtype=torch.bfloat16, device=dev)
    Vc = torch.empty((n_rows, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(K.decode_attend_workspace_bytes(1, n_rows, HQ, DH), dtype=torch.uint8, device=dev)
    # a plain copy of known size (outside the timed region): the reference for
    # scaling hardware byte counters (FETCH_SIZE / WRITE_SIZE) to bytes
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    del calib_src, calib_dst
    torch.cuda.synchronize()
    cursor = [N0 + WIN]
    ev = {k: [] for k in ("merge_k", "merge_v", "recon_kv", "attend")}
    attend_done = [None]
    # rows of every timed step: n_total (compressed + window) and the
    # compressed rows the K reconstruction kernel reads and writes (all rows
    # but the w-row exact window: every step folds the b rows that left it)
    timed_rows = []

    def step(record):
        s0 = cursor[0]
        n_total = s0 + BLK
        sk, sv = streams
        e = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        if attend_done[0] is not None:
            sv.wait_event(attend_done[0])  # the V factors and cache are rewritten only after the last step read them
        e[0].record(sk)
        if batched:
            ingest(s0, s0 + BLK)                 # K and V merges, one batched sequence (stream K)
            e[1].record(sk)
            sv.wait_event(e[1])
            e[3].record(sv)
            ev_vm = e[1]
        else:
            e[3].record(sv)
            wins[0].append(Xd[0][s0:s0 + BLK], s0)   # K merge (stream K)
            wins[1].append(Xd[1][s0:s0 + BLK], s0)   # V merge (stream V)
            e[1].record(sk)
            ev_vm = torch.cuda.Event(enable_timing=True)
            ev_vm.record(sv)
        # each path's exact window rows on its own stream (their positions are
        # disjoint from the compressed rows'), then the compressed rows of both
        # caches in one launch on stream K once both merges are done
        # (bracketed by e[5], e[2])
        for w_, C_, rope_, st_ in ((wins[0], Kc, True, sk), (wins[1], Vc, False, sv)):
            K.kv_scatter_exact(w_.rows, w_.pos, w_.rows.shape[0], D, n_total, DH, rope_, THETA, C_,
                               K.ISKV_OUT_BF16, st_)
        e[4].record(sv)
        sk.wait_event(e[4])
        e[5].record(sk)
        K.kv_reconstruct_batched([paths[0].h, paths[1].h], [Kc, Vc], [n_total, n_total], [True, False], DH, THETA,
                                 stream=sk)
        e[2].record(sk)
        e[7].record(sk)
        K.decode_attend(q, Kc, Vc, 1, n_total, HQ, HKV, DH, DH ** -0.5, o, ws, stream=sk)
        e[6].record(sk)
        attend_done[0] = e[6]
        if record:
            timed_rows.append((n_total, n_total - WIN))
            ev["merge_k"].append((e[0], e[1]))   # batched: the K + V merge sequence
            ev["merge_v"].append((e[3], ev_vm) if not batched else (e[0], e[1]))
            ev["recon_kv"].append((e[5], e[2]))
            ev["attend"].append((e[7], e[6]))
        cursor[0] += BLK

    for _ in range(warm):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # the bookkeeping behind timed_rows: after the last timed step the K
    # path holds every row but the window
    n_after = paths[0].n
    if n_after != timed_rows[-1][1]:
        raise RuntimeError(f"K path holds {n_after} compressed rows, expected {timed_rows[-1][1]}")

    def avg_ms(key):
        return float(np.mean([a.elapsed_time(b) for a, b in ev[key]]))

    # one history per launch: kv_reconstruct of the K path alone on its
    # stream, nothing else running (HIP events around each launch), beside
    # the step's two-path launch
    sk = streams[0]
    torch.cuda.synchronize()
    n_tot1, n_c1 = cursor[0], paths[0].n
    for _ in range(3):
        paths[0].reconstruct(Kc, n_tot1, head_dim=DH, rope=True, theta=THETA, stream=sk)
    es = [torch.cuda.Event(enable_timing=True) for _ in range(2 * SINGLE_REPS)]
    for i in range(SINGLE_REPS):
        es[2 * i].record(sk)
        paths[0].reconstruct(Kc, n_tot1, head_dim=DH, rope=True, theta=THETA, stream=sk)
        es[2 * i + 1].record(sk)
    sk.synchronize()
    s_ms = float(np.mean([es[2 * i].elapsed_time(es[2 * i + 1]) for i in range(SINGLE_REPS)]))
    s_bytes = n_c1 * R * 4 + R * D * 2 + n_c1 * D * 2
    single = {"ms": s_ms, "rows": n_c1, "algorithmic_bytes": s_bytes,
              "achieved_GBps": s_bytes / (s_ms * 1e-3) / 1e9, "frac": s_bytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
              "launches": SINGLE_REPS, "kernel": "kv_reconstruct (K path alone, bf16 + RoPE)"}

    # value side of the decode with the value history kept factored
    # (decode_attend_fv, outside the timed region) against the dense value
    # side of the timed step (V reconstruction + exact rows + attention over
    # rebuilt values), on the same caches
    torch.cuda.synchronize()
    n_tot = cursor[0]
    sv = streams[1]
    wsf = torch.empty(K.decode_attend_fv_workspace_bytes(paths[1].h, wins[1].rows.shape[0], HQ), dtype=torch.uint8,
                      device=dev)
    of = torch.empty((HQ, DH), dtype=torch.bfloat16, device=dev)
    ef = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    reps = 20

    def fv():
        K.decode_attend_fv(q[0], Kc, paths[1].h, wins[1].rows, wins[1].pos, wins[1].rows.shape[0], n_tot, HQ, HKV,
                           DH, DH ** -0.5, of, wsf, stream=sv)

    def dense_v():
        paths[1].reconstruct(Vc, n_tot, head_dim=DH, rope=False, stream=sv)
        K.kv_scatter_exact(wins[1].rows, wins[1].pos, wins[1].rows.shape[0], D, n_tot, DH, False, THETA, Vc,
                           K.ISKV_OUT_BF16, sv)
        K.decode_attend(q, Kc, Vc, 1, n_tot, HQ, HKV, DH, DH ** -0.5, o, ws, stream=sv)

    for _ in range(3):
        fv()
        dense_v()
    ef[0].record(sv)
    for _ in range(reps):
        fv()
    ef[1].record(sv)
    for _ in range(reps):
        dense_v()
    ef[2].record(sv)
    sv.synchronize()
    fv_ms = ef[0].elapsed_time(ef[1]) / reps
    dense_ms = ef[1].elapsed_time(ef[2]) / reps
    n_c = paths[1].n
    # algorithmic bytes: keys (n_total x D bf16), coordinates (n_c x k fp32), exact rows, basis
    fv_bytes = n_tot * D * 2 + n_c * R * 4 + wins[1].rows.shape[0] * D * 4 + D * R * 4
    fv_dev = float(np.abs(of.float().cpu().numpy() - o[0].float().cpu().numpy()).max())

    # stage breakdown of merges (outside the timed region): the handle runs
    # its merges kernel by kernel with HIP events at the stage boundaries; in
    # the batched layout each stage covers both paths (one launch per kernel)
    stage_runs = []
    n_before = []
    paths[0].set_timing(True)
    for _ in range(TIMED_MERGES):
        s0 = cursor[0]
        n_before.append(paths[0].n)
        if batched:
            ingest(s0, s0 + BLK)
        else:
            wins[0].append(Xd[0][s0:s0 + BLK], s0)
        stage_runs.append(paths[0].stage_times())
        cursor[0] += BLK
    paths[0].set_timing(False)
    torch.cuda.synchronize()
    stage_k = {k: float(np.mean([r[k] for r in stage_runs])) for k in stage_runs[0]}
    n_cu = float(np.mean(n_before))
    cu_paths = 2 if batched else 1
    # coordinate update of the old rows: read and write C (n x k fp32), 2 n k r flops, per path
    cu_bytes = cu_paths * 2.0 * n_cu * R * 4
    cu_gbps = cu_bytes / (stage_k["coord_update"] * 1e-3) / 1e9
    cu_tflops = cu_paths * 2.0 * n_cu * R * R / (stage_k["coord_update"] * 1e-3) / 1e12
    # the split-bf16 product runs three bf16 matrix-core products per output
    cu_bf16_frac = 3.0 * cu_tflops / BF16_PEAK_TFLOPS

    # merge modes on the K path, last because they change its factors: the
    # full merge (with its re-orthogonalisation every 256 rows), the
    # basis-only ablation (no coordinate rewrite) and the frozen basis (new
    # rows' coordinates only), MODE_MERGES merges each on the path's stream
    mode_ms = {}
    n_mode = paths[0].n
    pos_all = torch.arange(n_rows, dtype=torch.int32, device=dev)
    sk = streams[0]
    em = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def one_merge():
        s0 = cursor[0]
        paths[0].merge(Xd[0][s0:s0 + BLK], pos_all[s0:s0 + BLK])
        cursor[0] += BLK

    for name, mode in (("full", 0), ("basis_only", K.ISKV_NO_COORD_SYNC), ("frozen_basis", K.ISKV_FROZEN_BASIS)):
        paths[0].set_mode(mode)
        for _ in range(2):
            one_merge()
        em[0].record(sk)
        for _ in range(MODE_MERGES):
            one_merge()
        em[1].record(sk)
        sk.synchronize()
        mode_ms[name] = em[0].elapsed_time(em[1]) / MODE_MERGES

    ms = {k: avg_ms(k) for k in ev}
    core = [p.state() for p in paths]
    merges = 2 * steps
    # algorithmic bytes of the step's reconstruction launch (the K and the V
    # path), averaged over the timed steps: per path, read the n_c compressed
    # rows' coordinates (n_c x r fp32) and B^T (its bf16 copy, r x D), write
    # n_c x D bf16; flops 2 n_c r D per path. Both paths hold the same rows.
    n_c = float(np.mean([c for _, c in timed_rows]))
    recon_bytes = 2 * (n_c * R * 4 + R * D * 2 + n_c * D * 2)
    recon_flops = 2 * 2.0 * n_c * R * D
    recon_gbps = recon_bytes / (ms["recon_kv"] * 1e-3) / 1e9
    result = {
        "metric": "iSVD merges/s + reconstructed KV GB/s at n=16K, D=1024, r=256; % HBM/MFMA peak",
        "value": merges / dt,
        "unit": "merges/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": dt * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kv stream n=16384 (+decode), D=1024 (8x128), r=256, b=32, w=128, "
                               "K (exp(-i/40)+0.01) and V ((1+i)^-1/2) paths, bf16 RoPE reconstruction, "
                               "GQA 32q/8kv decode", "n_rows_start": N0, "rank": R, "block": BLK,
                   "window": WIN, "reorth_every_rows": 256, "hip_graphs": not args.no_graphs,
                   "kv_merges": "batched" if batched else "two streams"},
        "reconstructed_GBps": 2 * n_c * D * 2 / (ms["recon_kv"] * 1e-3) / 1e9,
        "timed_rows": {"n_total_first": timed_rows[0][0], "n_total_last": timed_rows[-1][0],
                       "compressed_mean": n_c},
        "stage_ms": ms,
        "host_issue_ms_per_step": t_issue * 1e3 / steps,
        "roofline": {"bound": "hbm", "achieved": recon_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": recon_gbps / HBM_PEAK_GBPS,
                     "traffic": profiled_traffic("recon_stream_kernel_kv_n16k_traffic.md"),
                     "algorithmic_bytes": recon_bytes,
                     "kernel": "kv_reconstruct_batched (K with RoPE and V, both paths in one launch, bf16)",
                     "paths_per_launch": 2,
                     "mfma_frac": recon_flops / (ms["recon_kv"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "recon_single_path": single,
        "merge_stage_ms": stage_k,
        "factor_v_attention": {"ms": fv_ms, "dense_value_side_ms": dense_ms, "algorithmic_bytes": fv_bytes,
                               "achieved_GBps": fv_bytes / (fv_ms * 1e-3) / 1e9, "n_total": n_tot,
                               "max_abs_vs_dense": fv_dev,
                               "split_kernel_traffic": profiled_traffic("fv_split_kernel_kv_n16k_traffic.md"),
                               "kernel": "decode_attend_fv (value history factored, no V reconstruction)"},
        "merge_stage_paths": cu_paths,
        "merge_modes": {"full_ms": mode_ms["full"], "basis_only_ms": mode_ms["basis_only"],
                        "frozen_basis_ms": mode_ms["frozen_basis"], "merges_each": MODE_MERGES,
                        "rows_at_start": n_mode,
                        "what": "K path alone on its stream, recorded sequences; full includes its "
                                "re-orthogonalisation every 256 rows; basis-only skips the coordinate "
                                "rewrite; frozen basis stores F B only"},
        "coord_update": {"bound": "hbm", "achieved": cu_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": cu_gbps / HBM_PEAK_GBPS, "algorithmic_bytes": cu_bytes, "rows": n_cu,
                         "traffic": profiled_traffic("xh_bf3s_kernel_coord_update_kv_n16k_traffic.md"),
                         "effective_tflops": cu_tflops, "bf16_mfma_frac": cu_bf16_frac,
                         "kernel": "xh_bf3s_kernel (old rows C <- C H[:k], streaming split-bf16 MFMA: 3 bf16 "
                                   "products, fp32 accumulation)",
                         "paths_per_launch": cu_paths, "merges_timed": TIMED_MERGES},
        "setup_s": {"generate": gen_s, "fill_16k_rows": fill_s},
        "core_solver_last_merge": [{"flags": c[11], "steps": c[12], "resid_sweeps": c[14], "k": c[1], "n": c[0]}
                                   for c in core],
    }
    if not args.main_only:
        result["coords_2byte"] = coords_leg(args, K, torch, dev, Xk, Kc)
        result["prefill_init"] = prefill_leg(args, K, torch, dev)
        result["prompt_decode_64k"] = prompt_decode_leg(args, K, torch, dev)
        if args.batch_paths > 0:
            result["batch_1024x32k"] = batch_leg(args, K, torch, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(Xk, Xv, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
