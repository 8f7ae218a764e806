#!/usr/bin/env python3
"""Benchmark of the retention hot path on one MI355X.

A step is one retention_chunkwise_fwd over the long workload (batch 1, 16
heads, L = 32768, d_k = 256, d_v = 512, bf16 inputs, chunk B = 512, xPos and
all three normalisations, bf16 output), the largest chunkwise configuration:
value = tokens/s = b*L / step time.  Its inputs (1.6 GB with the output) are
resident in HBM before timing and exceed the 256 MB MALL.  The same JSON line
carries, next to the headline, the medium workload (batch 4, 8 heads, L =
2048) at B = 512 (three rotated buffer sets, so the MALL cannot serve a
repeated set) and B = 64, each with its own roofline block; the decode step
(batch 128, 16 heads, 64 steps from position 8192) with its roofline block;
the measured ceilings (a streaming copy and an fp16 MFMA loop, both kernels of
this library); the parallel form on short sequences; the chunkwise backward;
the GroupNorm + gate epilogue; the gated MSR block (2 x 8192 tokens, d_model
4096), one RetNet layer around it and that layer decoding one token for 128
sequences; and the CPU legs of the fp64 oracle (chunkwise form, recurrent
form, decode step) on bounded samples of the same workloads.

Counter-derived figures (HBM bytes from FETCH_SIZE / WRITE_SIZE, MFMA busy
cycles) are read from the committed profiles/ summaries, and reported only
while the kernel sources hash to the value recorded there.

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
RIDGE = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
WARM_S = 0.05               # least untimed GPU work before a secondary leg is timed

CSRC = os.path.join("linear_attention_sequence_retention_amd", "csrc")
# the sources each profiled kernel group is built from
CHUNK_SOURCES = [os.path.join(CSRC, f) for f in ("chunk3.hip", "common.h", "internal.h")]
DECODE_SOURCES = [os.path.join(CSRC, f) for f in ("decode.hip", "common.h", "internal.h")]


def sources_sha256(files, root=ROOT):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profile_values(name, sources, root=ROOT):
    """The 'key: value' lines of a committed profiles/ summary, or {} when the
    file is missing or the kernel sources have changed since it was taken."""
    try:
        with open(os.path.join(root, "profiles", name)) as fh:
            text = fh.read()
    except OSError:
        return {}
    vals = dict(re.findall(r"^([a-z0-9_]+): (\S+)$", text, re.M))
    if vals.get("kernel_sources_sha256") != sources_sha256(sources, root):
        return {}
    return vals


def profiled_traffic(name, sources, root=ROOT):
    """HBM bytes per call from a FETCH_SIZE / WRITE_SIZE summary (copy-calibrated)."""
    v = profile_values(name, sources, root).get("traffic_bytes_per_call")
    return None if v is None else int(v)


def profiled_mfma(name, sources, root=ROOT):
    """MFMA busy fraction per kernel from a counter summary ({} if stale)."""
    vals = profile_values(name, sources, root)
    return {k[len("mfma_busy_"):]: float(v) for k, v in vals.items() if k.startswith("mfma_busy_")}


def roofline(flops, nbytes, ms, traffic):
    """The roofline block of a call: the binding roof by arithmetic intensity
    (algorithmic flops over compulsory bytes), achieved = algorithmic work /
    measured time."""
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    if flops / nbytes < RIDGE:
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    return {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_TFLOPS, 4), "traffic": traffic}


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


def time_calls(fn, n, warmup, torch, min_warm_s=0.0):
    """Average ms per call of fn() over n calls, HIP events on the stream the
    library launches on (torch's current stream), after `warmup` untimed calls
    and, for the secondary legs, as many more as fill min_warm_s seconds (after
    the host-side input generation between legs the GPU has idled, and the
    first tens of ms of work run slower than the steady state)."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_warm_s:
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


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, B, W, budget_s=10.0):
    """The fp64 oracle's chunkwise form (numpy + BLAS, all host threads) on a
    bounded sample of the headline workload: whole heads (every token of the
    sequence) one at a time until budget_s of CPU time has run; the rate is
    scaled to the whole workload (b*L tokens over h heads)."""
    import oracle
    q, k, v = W.chunkwise_inputs(**cfg)
    g, th = W.gamma_vector(cfg["h"]), W.theta_vector(cfg["dk"])
    t0 = time.perf_counter()
    heads = 0
    while True:
        bb, hh = divmod(heads % (cfg["b"] * cfg["h"]), cfg["h"])
        sl = (slice(bb, bb + 1), slice(hh, hh + 1))
        qs, ks, vs = (W.as_f32(a[sl], cfg["dtype"]).astype(np.float64) for a in (q, k, v))
        oracle.retention_chunkwise(qs, ks, vs, g[hh:hh + 1], th, cfg["flags"], B)
        heads += 1
        if time.perf_counter() - t0 > budget_s or heads >= 4 * cfg["b"] * cfg["h"]:
            break
    dt = (time.perf_counter() - t0) / heads                # per (batch, head) sequence
    total = dt * cfg["b"] * cfg["h"]
    return {"value": cfg["b"] * cfg["L"] / total, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"oracle.retention_chunkwise (fp64 numpy/BLAS, B={B}) over {heads} whole (batch, head) "
                      f"sequences of the {W.workload_name(cfg)} workload, {dt:.2f} s each; "
                      f"scaled to all {cfg['b'] * cfg['h']} heads"}


def cpu_legs(cfg, dec, W, budget_s=10.0):
    """The other CPU legs of the oracle: the recurrent form (the definition: a
    Python loop over positions, numpy over (batch, head)) on the first tokens
    of the headline workload, all heads, until budget_s; and the decode step on
    a few of the decode workload's sequences for its 64 steps (GB/s of fp32
    state read and written, the metric of the GPU leg)."""
    import oracle
    out = {"cores": _blas_threads()}
    q, k, v = W.chunkwise_inputs(**cfg)
    g, th = W.gamma_vector(cfg["h"]), W.theta_vector(cfg["dk"])
    n = 64
    while True:
        qs, ks, vs = (W.as_f32(a[:, :, :n], cfg["dtype"]).astype(np.float64) for a in (q, k, v))
        t0 = time.perf_counter()
        oracle.retention_recurrent(qs, ks, vs, g, th, cfg["flags"])
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or n >= cfg["L"]:
            break
        n = min(cfg["L"], n * 4)
    out["recurrent"] = {"value": cfg["b"] * n / dt, "unit": "tokens/s",
                        "sample": f"oracle.retention_recurrent over the first {n} tokens of every head of "
                                  f"{W.workload_name(cfg)}, {dt:.2f} s"}
    S0, qd, kd, vd = W.decode_inputs(**dec)
    gd, thd = W.gamma_vector(dec["h"]), W.theta_vector(dec["dk"])
    nb = 1
    while True:
        S = S0[:nb].astype(np.float64)
        t0 = time.perf_counter()
        for t in range(dec["steps"]):
            step_in = [W.as_f32(a[t, :nb], "bf16").astype(np.float64) for a in (qd, kd, vd)]
            _o, S, _z = oracle.recurrent_step(*step_in, S, gd, thd, dec["flags"], dec["pos0"] + t, dec["pos0"] + t + 1)
        dt = time.perf_counter() - t0
        if dt > budget_s / 4 or nb >= dec["b"]:
            break
        nb = min(dec["b"], nb * 4)
    state = nb * dec["h"] * dec["dk"] * dec["dv"] * 4
    out["decode"] = {"value": round(2 * state * dec["steps"] / dt / 1e9, 3), "unit": "GB/s",
                     "tokens_per_s": nb * dec["steps"] / dt,
                     "sample": f"oracle.recurrent_step, {nb} of {dec['b']} sequences x {dec['steps']} steps, "
                               f"{dt:.2f} s (fp32-equivalent state bytes read and written)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~20 calls on freshly placed inputs run ~9 % slower than the
    # steady state later calls settle at (20-step blocks on the long workload:
    # 1.27 ms, then 1.16-1.18 ms): the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true", help="time the primary workload only")
    ap.add_argument("--secondary",
                    default="medium,medium_B64,decode,ceilings,parallel_short,backward,gate_norm,block,layer,decode_layer",
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

    # ---- primary: the long workload, K timed steps bracketed by synchronisation
    lc = W.CHUNKWISE["long"]
    B = 512
    lq, lk, lv = W.chunkwise_inputs(**lc)
    lqd, lkd, lvd = dev(lq), dev(lk), dev(lv)
    del lq, lk, lv
    lo = torch.empty((lc["b"], lc["h"], lc["L"], lc["dv"]), dtype=torch.bfloat16, device="cuda")
    lg, lth = W.gamma_vector(lc["h"]), W.theta_vector(lc["dk"])
    lws = torch.empty(R.chunkwise_workspace_bytes(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"], B, lc["flags"]),
                      dtype=torch.uint8, device="cuda")

    def step():
        R.chunkwise_fwd(lqd, lkd, lvd, lg, lth, B, lc["flags"], out=lo, workspace=lws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_calls(step, args.steps, 0, torch)
    wall = time.perf_counter() - t0
    tokens = lc["b"] * lc["L"]
    value = tokens / (ms * 1e-3)
    flops = chunk_flops(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"], B)
    nbytes = chunk_bytes(lc["b"], lc["h"], lc["L"], lc["dk"], lc["dv"])
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = profiled_traffic("chunkwise_long_B512_traffic.md", CHUNK_SOURCES)
    roof = roofline(flops, nbytes, ms, traffic)
    extra = {"primary": {"kernel": "retention_chunkwise_fwd (delta, scan, output kernels)",
                         "arithmetic": "bf16 in and out, fp16 MFMA operands, fp32 accumulate",
                         "traffic_x_compulsory": None if traffic is None else round(traffic / nbytes, 2),
                         "mfma_busy": profiled_mfma("chunkwise_long_B512_mfma.md", CHUNK_SOURCES) or None,
                         "ms": round(ms, 4), "tflops": round(tflops, 1),
                         "mfma_frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
                         "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "alg_gflop": round(flops / 1e9, 2), "alg_mb": round(nbytes / 1e6, 1), "wall_s": round(wall, 3)}}
    del lqd, lkd, lvd, lo, lws
    torch.cuda.empty_cache()

    cfg = W.CHUNKWISE["medium"]
    b, h, L, dk, dv = cfg["b"], cfg["h"], cfg["L"], cfg["dk"], cfg["dv"]
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    flags = cfg["flags"]
    todo = set() if args.only_primary else set(x for x in args.secondary.split(",") if x)
    sets = []
    if todo & {"medium", "medium_B64", "backward"}:
        sets, _host = make_chunk_sets(cfg, 3, torch, W, dev)
        del _host
    it = [0]

    def mstep(Bc):
        qd, kd, vd, od = sets[it[0] % 3]
        it[0] += 1
        R.chunkwise_fwd(qd, kd, vd, g, th, Bc, flags, out=od)

    mtokens = b * L
    mbytes = chunk_bytes(b, h, L, dk, dv)
    for key, Bc, prof in (("medium", 512, "medium_B512"), ("medium_B64", 64, "medium_B64")):
        if key not in todo:
            continue
        # the medium workload, three rotated buffer sets (the MALL holds one)
        msm = time_calls(lambda: mstep(Bc), args.steps, args.warmup, torch, WARM_S)
        fl = chunk_flops(b, h, L, dk, dv, Bc)
        tr = profiled_traffic(f"chunkwise_{prof}_traffic.md", CHUNK_SOURCES)
        extra[key] = {"workload": "chunkwise_fwd " + W.workload_name(cfg, Bc), "ms": round(msm, 4),
                      "tokens_per_s": mtokens / (msm * 1e-3), "tflops": round(fl / (msm * 1e-3) / 1e12, 1),
                      "mfma_frac": round(fl / (msm * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                      "roofline": roofline(fl, mbytes, msm, tr),
                      "traffic_x_compulsory": None if tr is None else round(tr / mbytes, 2),
                      "mfma_busy": profiled_mfma(f"chunkwise_{prof}_mfma.md", CHUNK_SOURCES) or None}
    if "parallel_short" in todo:
        # short sequences (32 x 8 heads x 512 tokens, the medium head shape): the
        # parallel form (one chunk) against the chunkwise form at B = 64 and 128
        sb, sL = 32, 512
        sq, sk, sv = (dev(x) for x in W.chunkwise_inputs(sb, h, sL, dk, dv, "bf16", 1.0 / 16, seed=5))
        so = torch.empty((sb, h, sL, dv), dtype=torch.bfloat16, device="cuda")
        wsp = torch.empty(max(1, R.LIB.retention_parallel_workspace_bytes(sb, h, sL, dk, dv, 1, flags)),
                          dtype=torch.uint8, device="cuda")
        msp = time_calls(lambda: R.parallel_fwd(sq, sk, sv, g, th, flags, out=so, workspace=wsp), 10, args.warmup, torch, WARM_S)
        ent = {"parallel_ms": round(msp, 4), "tokens_per_s": sb * sL / (msp * 1e-3),
               "tflops": round(chunk_flops(sb, h, sL, dk, dv, sL) / (msp * 1e-3) / 1e12, 1)}
        for Bc in (64, 128):
            mc = time_calls(lambda: R.chunkwise_fwd(sq, sk, sv, g, th, Bc, flags, out=so), 10, args.warmup, torch, WARM_S)
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
                                                     dv=grads[2], workspace=wsb), max(5, args.steps // 2), max(2, args.warmup // 3), torch, WARM_S)
            fl = bwd_flops(b, h, L, dk, dv, Bb, True)
            ent = {"ms": round(msb, 4), "chunk": Bb, "tokens_per_s": mtokens / (msb * 1e-3),
                   "tflops": round(fl / (msb * 1e-3) / 1e12, 1),
                   "mfma_frac": round(fl / (msb * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4), "alg_gflop": round(fl / 1e9, 2)}
            if best is None or msb < best["ms"]:
                best = ent
            del wsb
        extra["backward"] = best
        del dod, grads
    del sets[:]
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
        msd = time_calls(decode64, 3, 1, torch, WARM_S) / dc["steps"]
        dbytes = 2 * db * dh * ddk * ddv * 4 + db * dh * (2 * ddk * 2 + ddv * 2 + ddv * 4)
        dflops = 4 * db * dh * ddk * ddv
        dtr = profiled_traffic("decode_b128_h16_traffic.md", DECODE_SOURCES)
        extra["decode"] = {"workload": "recurrent step b128 h16 dk256 dv512 fp32 state, 64 steps from position 8192",
                           "ms_per_step": round(msd, 4), "gbs": round(dbytes / (msd * 1e-3) / 1e9, 1),
                           "hbm_frac": round(dbytes / (msd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "tokens_per_s": db / (msd * 1e-3), "alg_mb_per_step": round(dbytes / 1e6, 1),
                           "roofline": roofline(dflops, dbytes, msd, dtr),
                           "traffic_x_compulsory": None if dtr is None else round(dtr / dbytes, 3)}
        del S, qd, kd, vd
        torch.cuda.empty_cache()
    if "ceilings" in todo:
        # measured ceilings from this library's own kernels: a 1 GiB streaming
        # copy (also the calibration kernel of the FETCH_SIZE / WRITE_SIZE
        # counters) and a loop of fp16 32x32x16 MFMAs on register operands
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        msc = time_calls(lambda: R.calib_copy(src, dst), 10, 2, torch, WARM_S)
        del src, dst
        nblk, iters = 4096, 2000
        mo = torch.empty(nblk * 256, dtype=torch.float32, device="cuda")
        msm_ = time_calls(lambda: R.calib_mfma(mo, nblk, iters), 5, 1, torch, WARM_S)
        mtf = nblk * 4 * iters * 4 * 32768 / (msm_ * 1e-3) / 1e12
        extra["ceilings"] = {"copy_1GiB": {"ms": round(msc, 4), "gbs": round(2 * (1 << 30) / (msc * 1e-3) / 1e9, 1),
                                           "frac_of_spec": round(2 * (1 << 30) / (msc * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                             "mfma_f16_loop": {"ms": round(msm_, 4), "tflops": round(mtf, 1),
                                               "frac_of_spec": round(mtf / PEAK_MFMA_TFLOPS, 4)}}
        del mo
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
                                                   bc["eps"]), 3, 1, torch, WARM_S)
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
        yc = W.LAYER
        msr_w, W1, W2, ln1, ln2 = W.layer_inputs(**yc)
        dT = lambda w: dev(np.ascontiguousarray(w.T))
        vec = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        Xd, ws, w1, w2 = dev(msr_w[0]), tuple(dT(w) for w in msr_w[1:]), dT(W1), dT(W2)
        l1, l2 = (vec(ln1[0]), vec(ln1[1])), (vec(ln2[0]), vec(ln2[1]))
        del msr_w, W1, W2
        lg, lth = W.gamma_vector(yc["h"]), W.theta_vector(yc["dk"])
        msl = time_calls(lambda: R.retnet_layer_fwd(Xd, ws, w1, w2, lg, lth, yc["chunk"], yc["flags"], yc["eps"],
                                                     yc["ln_eps"], l1, l2), 3, 1, torch, WARM_S)
        M, dm, hdk, hdv, dff = yc["b"] * yc["L"], yc["d_model"], yc["h"] * yc["dk"], yc["h"] * yc["dv"], yc["d_ff"]
        gflop = 2 * M * dm * (2 * hdk + 2 * hdv) + 2 * M * hdv * dm + 4 * M * dm * dff
        rflop = chunk_flops(yc["b"], yc["h"], yc["L"], yc["dk"], yc["dv"], yc["chunk"])
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
                                                       dc["ln_eps"]), 10, 2, torch, WARM_S)
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
        msg = time_calls(lambda: R.gate_norm(y, gg, 1e-5, out=zo), 20, args.warmup, torch, WARM_S)
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
        "config": {"workload": "chunkwise_fwd " + W.workload_name(lc, B) + " xpos+all_norms",
                   "global_batch": lc["b"], "seq_len": lc["L"], "heads": lc["h"], "d_k": lc["dk"], "d_v": lc["dv"],
                   "chunk": B, "parallelism": "single_gpu"},
        "roofline": roof,
        "mfma": {"achieved": round(tflops, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / PEAK_MFMA_TFLOPS, 4)},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(lc, B, W)
        extra["cpu_legs"] = cpu_legs(lc, W.DECODE, W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
