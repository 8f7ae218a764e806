#!/usr/bin/env python3
"""Benchmark of the retention hot path on one MI355X.

A step is one retention_chunkwise_fwd over the medium workload (batch 4, 8
heads, L = 2048, d_k = 256, d_v = 512, bf16 inputs, chunk B = 512, xPos and all
three normalisations, bf16 output): value = tokens/s = b*L / step time.  The
inputs are resident in HBM before timing; three input/output buffer sets are
rotated so the 256 MB MALL cannot serve a repeated set.  Secondary lines in
the same JSON record: the same workload at B = 64, the long workload (L =
32768, 16 heads), the parallel form on short sequences (32 x 8 heads x 512)
against the chunkwise form, the chunkwise backward on the medium workload, the decode
step (batch 128, 16 heads, 64 steps from
position 8192), the GroupNorm + gate epilogue at the block shape, the gated
MSR block (2 x 8192 tokens, d_model 4096), one RetNet layer around it
(LayerNorms, residuals and a 4 x d_model gelu FFN), and that layer decoding
one token for 128 sequences.

Prints ONE JSON line.  Only N = 1 GPU is supported.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# counter summary of the primary step and the sources its kernels are built from
TRAFFIC_PROFILE = os.path.join("profiles", "chunkwise_medium_B512_traffic.md")
TRAFFIC_SOURCES = [os.path.join("linear_attention_sequence_retention_amd", "csrc", f)
                   for f in ("chunk3.hip", "common.h", "internal.h")]


def sources_sha256(root=ROOT):
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(root=ROOT):
    """HBM bytes per call of the primary step from the committed FETCH_SIZE /
    WRITE_SIZE summary (copy-calibrated), or None when the kernel sources have
    changed since the counters were taken."""
    try:
        with open(os.path.join(root, TRAFFIC_PROFILE)) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_call|kernel_sources_sha256): (\S+)$", text, re.M))
    if vals.get("kernel_sources_sha256") != sources_sha256(root) or "traffic_bytes_per_call" not in vals:
        return None
    return int(vals["traffic_bytes_per_call"])


def chunk_flops(b, h, L, dk, dv, B, with_state_out=False):
    """Algorithmic flops of the chunkwise form: causal half of the intra-chunk
    scores and P.V, the cross term for chunks >= 1 and the state update for
    chunks that feed a later chunk (plus the last one when the state is
    written out)."""
    nc = (L + B - 1) // B
    intra = sum(min(B, L - c * B) * (min(B, L - c * B) + 1) * (dk + dv) for c in range(nc))
    cross = (nc - 1) * 2 * B * dk * dv
    state = (nc - 1 + (1 if with_state_out else 0)) * 2 * B * dk * dv
    return b * h * (intra + cross + state)


def bwd_flops(b, h, L, dk, dv, B, score_norm):
    """Algorithmic flops of the chunkwise backward, each product counted once:
    the causal half of the intra-chunk products Q'K'^T and dO V^T, E K',
    E^T Q' and (a A)^T dO; the cross terms dO R^T (chunks >= 1), V U^T and
    K' U (chunks before the last); and the two state scans K'^T (zeta V) and
    Q'^T (w dO).  The score normalisation's row statistics add no product:
    (q' R) . dO is q' . (dO R^T), a row dot product of a term dq needs anyway.
    score_norm is kept for the signature."""
    nc = (L + B - 1) // B
    pairs = sum(min(B, L - c * B) * (min(B, L - c * B) + 1) // 2 for c in range(nc))
    intra = 2 * pairs * ((dk + dv) + (2 * dk + dv))
    rows_after_first = max(L - B, 0)
    rows_before_last = L - min(B, L - (nc - 1) * B)
    cross = 2 * dk * dv * (rows_after_first + 2 * rows_before_last)
    states = 2 * 2 * L * dk * dv
    return b * h * (intra + cross + states)


def chunk_bytes(b, h, L, dk, dv, in_bytes=2, out_bytes=2):
    return b * h * L * (2 * dk * in_bytes + dv * in_bytes + dv * out_bytes)


def time_calls(fn, n, warmup, torch):
    """Average ms per call of fn() over n calls, HIP events on the stream the
    library launches on (torch's current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(n):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def make_chunk_sets(cfg, nsets, torch, W, dev):
    q, k, v = W.chunkwise_inputs(**cfg)
    sets = []
    for s in range(nsets):
        sets.append((dev(q), dev(k), dev(v),
                     torch.empty((cfg["b"], cfg["h"], cfg["L"], cfg["dv"]), dtype=torch.bfloat16, device="cuda")))
    return sets, (q, k, v)


def cpu_baseline(cfg, B, W):
    """The fp64 oracle (chunkwise form, numpy + BLAS) on the medium workload
    (all four sequences, all heads, full L), repeated until at least 10 s of
    CPU time has run; tokens/s over the runs."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    q, k, v = W.chunkwise_inputs(**cfg)
    qs, ks, vs = (W.as_f32(a, cfg["dtype"]).astype(np.float64) for a in (q, k, v))
    g, th = W.gamma_vector(cfg["h"]), W.theta_vector(cfg["dk"])
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.retention_chunkwise(qs, ks, vs, g, th, cfg["flags"], B)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 200:
            break
    dt = (time.perf_counter() - t0) / reps
    toks = cfg["b"] * cfg["L"]
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.retention_chunkwise (fp64 numpy/BLAS) over the whole medium workload "
                      f"(b={cfg['b']}, {cfg['h']} heads, L={cfg['L']}, B={B}), {reps} run(s) of {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true", help="time the primary workload only")
    ap.add_argument("--secondary", default="medium_B64,parallel_short,backward,long,decode,gate_norm,block,layer,decode_layer,copy",
                    help="comma list of secondary measurements to run (empty for none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path is single-GPU "
              "and its multi-GPU sharding is a design note, not a measured mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_sequence_retention_amd import binding as R
    from linear_attention_sequence_retention_amd import workloads as W

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    cfg = W.CHUNKWISE["medium"]
    b, h, L, dk, dv = cfg["b"], cfg["h"], cfg["L"], cfg["dk"], cfg["dv"]
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    flags = cfg["flags"]
    B = 512
    sets, host = make_chunk_sets(cfg, 3, torch, W, dev)
    it = [0]

    def step(Bc=B):
        qd, kd, vd, od = sets[it[0] % 3]
        it[0] += 1
        R.chunkwise_fwd(qd, kd, vd, g, th, Bc, flags, out=od)

    # ---- primary: K timed steps bracketed by synchronisation
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_kernel = time_calls(step, args.steps, 0, torch)
    wall = time.perf_counter() - t0
    ms = ms_kernel
    tokens = b * L
    value = tokens / (ms * 1e-3)
    flops = chunk_flops(b, h, L, dk, dv, B)
    nbytes = chunk_bytes(b, h, L, dk, dv)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    intensity = flops / nbytes
    ridge = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "hbm" if intensity < ridge else "mfma"
    traffic = profiled_traffic()
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "traffic": traffic}

    extra = {"primary": {"kernel": "retention_chunkwise_fwd (delta, scan, output kernels)",
                         "arithmetic": "bf16 in and out, fp16 MFMA operands, fp32 accumulate",
                         "traffic_x_compulsory": None if traffic is None else round(traffic / nbytes, 2),
                         "ms": round(ms, 4), "tflops": round(tflops, 1),
                         "mfma_frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "gbs": round(gbs, 1),
                         "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "alg_gflop": round(flops / 1e9, 2),
                         "alg_mb": round(nbytes / 1e6, 1), "wall_s": round(wall, 3)}}

    todo = set() if args.only_primary else set(x for x in args.secondary.split(",") if x)
    if "medium_B64" in todo:
        # same workload at B = 64
        ms64 = time_calls(lambda: step(64), max(5, args.steps // 2), 2, torch)
        f64_ = chunk_flops(b, h, L, dk, dv, 64)
        extra["medium_B64"] = {"ms": round(ms64, 4), "tokens_per_s": tokens / (ms64 * 1e-3),
                               "tflops": round(f64_ / (ms64 * 1e-3) / 1e12, 1),
                               "mfma_frac": round(f64_ / (ms64 * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                               "gbs": round(nbytes / (ms64 * 1e-3) / 1e9, 1)}
    if "parallel_short" in todo:
        # short sequences (32 x 8 heads x 512 tokens, the medium head shape): the
        # parallel form (one chunk) against the chunkwise form at B = 64 and 128
        sb, sL = 32, 512
        sq, sk, sv = (dev(x) for x in W.chunkwise_inputs(sb, h, sL, dk, dv, "bf16", 1.0 / 16, seed=5))
        so = torch.empty((sb, h, sL, dv), dtype=torch.bfloat16, device="cuda")
        wsp = torch.empty(max(1, R.LIB.retention_parallel_workspace_bytes(sb, h, sL, dk, dv, 1, flags)),
                          dtype=torch.uint8, device="cuda")
        msp = time_calls(lambda: R.parallel_fwd(sq, sk, sv, g, th, flags, out=so, workspace=wsp), 10, 3, torch)
        ent = {"parallel_ms": round(msp, 4), "tokens_per_s": sb * sL / (msp * 1e-3),
               "tflops": round(chunk_flops(sb, h, sL, dk, dv, sL) / (msp * 1e-3) / 1e12, 1)}
        for Bc in (64, 128):
            mc = time_calls(lambda: R.chunkwise_fwd(sq, sk, sv, g, th, Bc, flags, out=so), 10, 3, torch)
            ent[f"chunkwise_B{Bc}_ms"] = round(mc, 4)
        extra["parallel_short"] = ent
        del sq, sk, sv, so, wsp
    if "backward" in todo:
        # chunkwise backward on the medium workload (dq, dk, dv in fp32 from a bf16 dO)
        qd, kd, vd, _ = sets[0]
        rng = np.random.default_rng(77)
        dod = dev(W.draw(rng, (b, h, L, dv), 1.0, "bf16"))
        grads = [torch.empty((b, h, L, dk), device="cuda"), torch.empty((b, h, L, dk), device="cuda"),
                 torch.empty((b, h, L, dv), device="cuda")]
        best = None
        for Bb in (256, 512):
            wsb = torch.empty(R.chunkwise_bwd_workspace_bytes(b, h, L, dk, dv, Bb), dtype=torch.uint8, device="cuda")
            msb = time_calls(lambda: R.chunkwise_bwd(qd, kd, vd, dod, g, th, Bb, flags, dq=grads[0], dk=grads[1],
                                                     dv=grads[2], workspace=wsb), max(5, args.steps // 2), 2, torch)
            fl = bwd_flops(b, h, L, dk, dv, Bb, True)
            ent = {"ms": round(msb, 4), "chunk": Bb, "tokens_per_s": tokens / (msb * 1e-3),
                   "tflops": round(fl / (msb * 1e-3) / 1e12, 1),
                   "mfma_frac": round(fl / (msb * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4), "alg_gflop": round(fl / 1e9, 2)}
            if best is None or msb < best["ms"]:
                best = ent
            del wsb
        extra["backward"] = best
        del dod, grads
    del sets[:]
    torch.cuda.empty_cache()
    if "long" in todo:
        # long workload
        lc = W.CHUNKWISE["long"]
        lq, lk, lv = W.chunkwise_inputs(**lc)
        lqd, lkd, lvd = dev(lq), dev(lk), dev(lv)
        del lq, lk, lv
        lo = torch.empty((lc["b"], lc["h"], lc["L"], lc["dv"]), dtype=torch.bfloat16, device="cuda")
        lg, lth = W.gamma_vector(lc["h"]), W.theta_vector(lc["dk"])
        msl = time_calls(lambda: R.chunkwise_fwd(lqd, lkd, lvd, lg, lth, 512, lc["flags"], out=lo), 3, 1, torch)
        fl = chunk_flops(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"], 512)
        bl = chunk_bytes(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"])
        extra["long_B512"] = {"ms": round(msl, 3), "tokens_per_s": lc["b"] * lc["L"] / (msl * 1e-3),
                              "tflops": round(fl / (msl * 1e-3) / 1e12, 1),
                              "mfma_frac": round(fl / (msl * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                              "gbs": round(bl / (msl * 1e-3) / 1e9, 1)}
        del lqd, lkd, lvd, lo
        torch.cuda.empty_cache()
    if "decode" in todo:
        # decode: 64 sequential steps at batch 128
        dc = W.DECODE
        db, dh, ddk, ddv = dc["b"], dc["h"], dc["dk"], dc["dv"]
        S0, qs, ks, vs = W.decode_inputs(**dc)
        S = torch.from_numpy(S0).cuda()
        del S0
        qd = [dev(x) for x in qs]
        kd = [dev(x) for x in ks]
        vd = [dev(x) for x in vs]
        od = torch.empty((db, dh, ddv), dtype=torch.float32, device="cuda")
        dg, dth = W.gamma_vector(dh), W.theta_vector(ddk)
        pos0 = dc["pos0"]

        def decode64():
            for t in range(dc["steps"]):
                R.recurrent_step(qd[t], kd[t], vd[t], S, dg, dth, pos0 + t, pos0 + t + 1, dc["flags"], out=od)
        msd = time_calls(decode64, 3, 1, torch) / dc["steps"]
        dbytes = 2 * db * dh * ddk * ddv * 4 + db * dh * (2 * ddk * 2 + ddv * 2 + ddv * 4)
        extra["decode"] = {"ms_per_step": round(msd, 4), "gbs": round(dbytes / (msd * 1e-3) / 1e9, 1),
                           "hbm_frac": round(dbytes / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "tokens_per_s": db / (msd * 1e-3), "alg_mb_per_step": round(dbytes / 1e6, 1)}
        del S, qd, kd, vd
        torch.cuda.empty_cache()
    if "copy" in todo:
        # a plain 1 GiB device copy: measured HBM reference and the
        # calibration kernel for the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        msc = time_calls(lambda: dst.copy_(src), 5, 1, torch)
        extra["copy_1GiB"] = {"ms": round(msc, 4), "gbs": round(2 * (1 << 30) / (msc * 1e-3) / 1e9, 1)}
        del src, dst
        torch.cuda.empty_cache()
    if "block" in todo:
        # full gated MSR block forward: 2 x 8192 tokens, d_model 4096, 16 heads
        bc = W.BLOCK
        X, WQ, WK, WV, WG, WO = W.block_inputs(**bc)
        dT = lambda w: dev(np.ascontiguousarray(w.T))
        Xd, wq, wk, wv, wg, wo = dev(X), dT(WQ), dT(WK), dT(WV), dT(WG), dT(WO)
        del X, WQ, WK, WV, WG, WO
        bg, bth = W.gamma_vector(bc["h"]), W.theta_vector(bc["dk"])
        msb = time_calls(lambda: R.msr_block_fwd(Xd, wq, wk, wv, wg, wo, bg, bth, bc["chunk"], bc["flags"],
                                                   bc["eps"]), 3, 1, torch)
        M, dm, hdk, hdv = bc["b"] * bc["L"], bc["d_model"], bc["h"] * bc["dk"], bc["h"] * bc["dv"]
        gflop = 2 * M * dm * (2 * hdk + 2 * hdv) + 2 * M * hdv * dm
        rflop = chunk_flops(bc["b"], bc["h"], bc["L"], bc["dk"], bc["dv"], bc["chunk"])
        extra["block"] = {"ms": round(msb, 3), "tokens_per_s": M / (msb * 1e-3),
                          "tflops": round((gflop + rflop) / (msb * 1e-3) / 1e12, 1),
                          "gemm_gflop": round(gflop / 1e9, 1), "retention_gflop": round(rflop / 1e9, 1)}
        del Xd, wq, wk, wv, wg, wo
        torch.cuda.empty_cache()
    if "layer" in todo:
        # one RetNet layer around the block: LN, MSR + residual, LN, FFN (4 x d_model, gelu) + residual
        lc = W.LAYER
        msr_w, W1, W2, ln1, ln2 = W.layer_inputs(**lc)
        dT = lambda w: dev(np.ascontiguousarray(w.T))
        vec = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        Xd, ws, w1, w2 = dev(msr_w[0]), tuple(dT(w) for w in msr_w[1:]), dT(W1), dT(W2)
        l1, l2 = (vec(ln1[0]), vec(ln1[1])), (vec(ln2[0]), vec(ln2[1]))
        del msr_w, W1, W2
        lg, lth = W.gamma_vector(lc["h"]), W.theta_vector(lc["dk"])
        msl = time_calls(lambda: R.retnet_layer_fwd(Xd, ws, w1, w2, lg, lth, lc["chunk"], lc["flags"], lc["eps"],
                                                     lc["ln_eps"], l1, l2), 3, 1, torch)
        M, dm, hdk, hdv, dff = lc["b"] * lc["L"], lc["d_model"], lc["h"] * lc["dk"], lc["h"] * lc["dv"], lc["d_ff"]
        gflop = 2 * M * dm * (2 * hdk + 2 * hdv) + 2 * M * hdv * dm + 4 * M * dm * dff
        rflop = chunk_flops(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"], lc["chunk"])
        extra["layer"] = {"ms": round(msl, 3), "tokens_per_s": M / (msl * 1e-3),
                          "tflops": round((gflop + rflop) / (msl * 1e-3) / 1e12, 1), "d_ff": dff,
                          "gemm_gflop": round(gflop / 1e9, 1), "retention_gflop": round(rflop / 1e9, 1)}
        del Xd, ws, w1, w2
        torch.cuda.empty_cache()
    if "decode_layer" in todo:
        # one RetNet layer decoding one token for 128 sequences (d_model 4096, 16 heads, FFN 16384)
        dc = dict(W.LAYER, b=128, L=1)
        msr_w, W1, W2, ln1, ln2 = W.layer_inputs(**dc)
        dT = lambda w: dev(np.ascontiguousarray(w.T))
        vec = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        lay = [(tuple(dT(w) for w in msr_w[1:]), dT(W1), dT(W2), (vec(ln1[0]), vec(ln1[1])),
                (vec(ln2[0]), vec(ln2[1])))]
        del msr_w, W1, W2
        db, dh, ddk, ddv, ddm, dff = dc["b"], dc["h"], dc["dk"], dc["dv"], dc["d_model"], dc["d_ff"]
        st = R.new_states(1, db, dh, ddk, ddv)
        xd = torch.randn((db, ddm), device="cuda")
        dg, dth = W.gamma_vector(dh), W.theta_vector(ddk)
        msd = time_calls(lambda: R.retnet_decode_step(xd, lay, st, dg, dth, 8192, 8193, dc["flags"], dc["eps"],
                                                       dc["ln_eps"]), 10, 2, torch)
        wbytes = 2 * (ddm * (2 * dh * ddk + 2 * dh * ddv) + dh * ddv * ddm + 2 * ddm * dff)
        sbytes = 2 * 4 * db * dh * ddk * ddv
        extra["decode_layer"] = {"ms": round(msd, 4), "tokens_per_s": db / (msd * 1e-3),
                                 "weight_mb": round(wbytes / 1e6, 1), "state_mb": round(sbytes / 1e6, 1),
                                 "gbs": round((wbytes + sbytes) / (msd * 1e-3) / 1e9, 1),
                                 "hbm_frac": round((wbytes + sbytes) / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del lay, st
        torch.cuda.empty_cache()
    if "gate_norm" in todo:
        # GroupNorm + gate at the block shape (2 x 8192 tokens, 16 heads x 512)
        gb, gL, gh, gdv = 2, 8192, 16, 512
        y = torch.randn((gb, gh, gL, gdv), device="cuda").to(torch.bfloat16)
        gg = torch.randn((gb, gL, gh * gdv), device="cuda").to(torch.bfloat16)
        zo = torch.empty_like(gg)
        msg = time_calls(lambda: R.gate_norm(y, gg, 1e-5, out=zo), 20, 3, torch)
        gbytes = 3 * gb * gL * gh * gdv * 2
        extra["gate_norm"] = {"ms": round(msg, 4), "gbs": round(gbytes / (msg * 1e-3) / 1e9, 1),
                              "hbm_frac": round(gbytes / (msg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    line = {
        "metric": "chunkwise retention fwd tokens/s & % bf16 MFMA peak; decode step GB/s % HBM",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "chunkwise_fwd " + W.workload_name(cfg, B) + " xpos+all_norms",
                   "global_batch": b, "seq_len": L, "heads": h, "d_k": dk, "d_v": dv, "chunk": B,
                   "parallelism": "single_gpu"},
        "roofline": roof,
        "mfma": {"achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / PEAK_MFMA_TFLOPS, 4)},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, B, W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
