#!/usr/bin/env python3
"""Batch-1 decode benchmark of the persistent engine on one MI355X.

Workloads: the DeepSeek-V3-shaped stack of 3 dense + 8 MoE MLA layers with a
bf16 LM head (vocabulary 129,280), FP8-e4m3 weights with 128x128 bf16 block
scales, batch 1, a prompt cache of synthetic N(0,1) bf16 latents, and 1024
teacher-forced decode steps of seeded random token ids (the pages' InferenceX
1k/1k and 8k/1k sequence lengths; no dataset). The headline workload is
dsv3_stack_1k (cache 1025 -> 2048 rows); dsv3_stack_8k (8193 -> 9216) is
measured in the same run on the same engine and weights.

Each workload is timed two ways, both with HIP events on the launch stream and
inputs resident in HBM: K back-to-back single-step launches, and one resident
launch of the same K steps (the engine stays on the device for the whole
request; this is the headline figure). Then the bare DeepSeek-V3-shaped dense
and MoE layers are timed per layer-step, alternating over two weight copies so
that no step is served from the MALL, and the weight products of one MoE layer
are timed at batch 1, 2, 4 and 8 (pdm_batch_gemm / pdm_batch_ffn, several
sequences sharing every weight byte), as are whole batched decode steps of the
stack (pdm_batch_decode_step). Sparse (DSA) attention of one DeepSeek-V3
layer (indexer, top-2048, attention over the chosen rows) is timed at cache
lengths 9216, 32768 and 131072. Prints one JSON line with tok/s/user, TPOT, the
HBM roofline fraction, a stage trace, the single-layer timings, the batch
points, the sparse-attention points and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import math
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

SEED = 0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def engine_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("engine.hip", "pdm_internal.h", "planner.cpp"):
        with open(os.path.join(ROOT, "persistent_decode_megakernel_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def git_head() -> str:
    try:
        return subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"], capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def load_traffic(workload: str):
    """HBM traffic per step from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"engine_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("engine_source_hash") != engine_source_hash():
        return None
    return d.get("hbm_bytes_per_step")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, store, pos):
    """Time the CPU oracle on a bounded sample of one decode step: one dense
    layer, one MoE layer and 1/16 of the LM head rows, then extrapolate to a
    whole token (3 dense + 8 MoE layers + the full LM head)."""
    import numpy as np
    import oracle as O
    from oracle import model as M
    from synth import gen
    W = O.OracleWeights(store, cache_limit_bytes=0)
    st = O.DecodeState.empty(cfg, pos + 1)
    dense_l = cfg.layers.index("dense")
    moe_l = cfg.layers.index("moe")
    for l in (dense_l, moe_l):
        rows = gen.latent_rows(cfg, l, pos, SEED, device=store.device).cpu().numpy().view(np.uint16)
        st.cache[l][:pos] = O.bf16_bits_to_f64(rows)
    x = W.bf16_row("embed", gen.decode_token(cfg, 0, 0, SEED))
    t = {}
    for name, l in (("dense", dense_l), ("moe", moe_l)):
        t0 = time.perf_counter()
        x = M.attention_decode(W, cfg, l, x, pos, st, True)
        x = O.bf16_round(M.ffn_decode(W, cfg, l, x))
        t[name] = time.perf_counter() - t0
        log(f"cpu baseline: oracle {name} layer {t[name]:.2f} s")
    t0 = time.perf_counter()
    lm = store.numpy("lm_head")["data"]
    rows = lm.shape[0] // 16
    hf = O.rmsnorm(x, W("final_norm"), cfg.rms_eps)
    _ = O.bf16_bits_to_f64(lm[:rows]) @ hf
    t["lm_sixteenth"] = time.perf_counter() - t0
    n_dense, n_moe = cfg.layers.count("dense"), cfg.layers.count("moe")
    per_token = n_dense * t["dense"] + n_moe * t["moe"] + 16 * t["lm_sixteenth"]
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info}))
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return {"value": 1.0 / per_token, "unit": "tok/s/user", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "extrapolated": True,
            "sample": (f"float64 numpy oracle timed on one dense layer ({t['dense']:.2f} s), one MoE layer "
                       f"({t['moe']:.2f} s) and 1/16 of the LM head rows ({t['lm_sixteenth']:.2f} s) of one "
                       f"decode step at context {pos + 1}; extrapolated to {n_dense} dense + {n_moe} MoE layers + "
                       f"the full LM head = {per_token:.1f} s per token"),
            "cpu_model": cpu_model(), "blas": blas, "blas_threads": threads, "seed": SEED}


def stream_ceiling(buf, nbytes: int = 32 << 30) -> float:
    """Achievable HBM read rate of a plain streaming kernel on this GPU: a sum
    over nbytes of the (already resident) weight arena, best of 3."""
    import torch
    n = min(nbytes, buf.numel()) // 16 * 16
    v = buf[:n].view(torch.int64)
    best = None
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        v.sum()
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / 1e3
        best = s if best is None else min(best, s)
    return n / best


def calibrate_copy(nbytes: int = 1 << 30):
    """A plain device-to-device copy of a known size, for scaling the HBM byte
    counters of rocprofv3 (FETCH_SIZE, WRITE_SIZE) to bytes: run it under the
    same counter as the engine and divide the known bytes by the reading."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "copies": 3}), flush=True)


def run_workload(eng, cfg, K, Wm, do_trace, trace_detail, resident_only=False):
    """Time K teacher-forced steps of cfg on the bound engine, as K single-step
    launches and as one resident launch (resident_only: only the resident
    warm-up and timed launches, so that every engine launch of the process
    runs many steps — for profiler runs). Returns a result dict."""
    import torch
    from persistent_decode_megakernel_amd import describe_plan, roofline as R, trace as T
    from synth import gen
    P = cfg.prompt_len
    lat = [gen.latent_rows(cfg, l, P, SEED, device="cuda") for l in range(cfg.n_layers)]
    toks = [gen.decode_token(cfg, j, 0, SEED) for j in range(max(K, Wm))]
    tok_dev = torch.tensor(toks, dtype=torch.int32, device="cuda")
    am = torch.zeros(max(K, Wm), dtype=torch.int32, device="cuda")

    def fill():
        eng.reset()
        for l in range(cfg.n_layers):
            eng.import_kv(l, 0, lat[l])

    stream = torch.cuda.current_stream()
    if not resident_only:
        fill()
        for j in range(Wm):
            eng.decode(P + j, token=toks[j])
        rc, st = eng.status()
        if rc != 0:
            raise SystemExit(f"{cfg.name}: warm-up step failed: status {rc} stage {st.stage}")
    fill()
    eng.decode_steps(P, tok_dev[:Wm].clone(), argmax=am[:Wm])
    rc, st = eng.status()
    if rc != 0:
        raise SystemExit(f"{cfg.name}: resident warm-up failed: status {rc} stage {st.stage}")

    # K single-step launches
    if not resident_only:
        fill()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev[0].record(stream)
        for j in range(K):
            eng.decode(P + j, token=toks[j])
            ev[j + 1].record(stream)
        torch.cuda.synchronize()
        rc, st = eng.status()
        if rc != 0:
            raise SystemExit(f"{cfg.name}: timed step failed: status {rc} stage {st.stage}")
        per = sorted(ev[j].elapsed_time(ev[j + 1]) for j in range(K))
        launch_s = ev[0].elapsed_time(ev[K]) / 1e3 / K

    # one resident launch of the same K steps
    fill()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    eng.decode_steps(P, tok_dev[:K], argmax=am[:K])
    e1.record(stream)
    torch.cuda.synchronize()
    rc, st = eng.status()
    if rc != 0:
        raise SystemExit(f"{cfg.name}: resident launch failed: status {rc} stage {st.stage}")
    resident_s = e0.elapsed_time(e1) / 1e3 / K

    # the same resident launch decoding greedily: each step's token is the
    # previous step's argmax, fed back on the device (autoregressive decode)
    greedy_s = None
    if cfg.vocab > 0 and not resident_only:
        fill()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        eng.decode_steps(P, tok_dev[:1].clone(), n_steps=K, greedy=True, argmax=am[:K])
        g1.record(stream)
        torch.cuda.synchronize()
        rc, st = eng.status()
        if rc != 0:
            raise SystemExit(f"{cfg.name}: greedy resident launch failed: status {rc} stage {st.stage}")
        greedy_s = g0.elapsed_time(g1) / 1e3 / K

    bytes_mean = R.mean_bytes_per_token(cfg, P, K)
    out = {
        "workload": cfg.name, "prompt_positions": P, "context_range": [P + 1, P + K], "steps": K,
        "bytes_per_token": int(bytes_mean),
        "resident": {"ms_per_step": round(resident_s * 1e3, 4), "tok_s_user": round(1 / resident_s, 3),
                     "frac_of_8TBps": round(bytes_mean / resident_s / R.HBM_PEAK_BYTES_PER_S, 4)},
    }
    if greedy_s is not None:
        out["resident_greedy"] = {"ms_per_step": round(greedy_s * 1e3, 4), "tok_s_user": round(1 / greedy_s, 3),
                                  "frac_of_8TBps": round(bytes_mean / greedy_s / R.HBM_PEAK_BYTES_PER_S, 4),
                                  "tokens": "each step's argmax, fed back on the device"}
    if not resident_only:
        out["per_step_launch"] = {"ms_per_step": round(launch_s * 1e3, 4), "tok_s_user": round(1 / launch_s, 3),
                                  "p50_ms": round(per[K // 2], 4), "p99_ms": round(per[min(K - 1, int(0.99 * K))], 4),
                                  "frac_of_8TBps": round(bytes_mean / launch_s / R.HBM_PEAK_BYTES_PER_S, 4)}
    log(f"{cfg.name}: resident {resident_s * 1e3:.3f} ms/token ({1 / resident_s:.1f} tok/s/user, "
        f"{bytes_mean / resident_s / 1e9:.0f} GB/s)"
        + ("" if resident_only else f"; single-step launches {launch_s * 1e3:.3f} ms/token")
        + ("" if greedy_s is None else f"; greedy resident {greedy_s * 1e3:.3f} ms/token"))
    if do_trace:
        plan = describe_plan(cfg, eng.max_ctx, eng.sizes.n_workgroups)
        fill()
        eng.set_trace(True)
        sums, traces = [], []
        for j in range(4):
            eng.decode(P + j, token=toks[j])
            eng.status()
            traces.append(eng.taps()["trace"].cpu().numpy().copy())
            sums.append(T.summarize(traces[-1], plan))
        eng.set_trace(False)
        bi = min(range(len(sums)), key=lambda i: sums[i]["total_us"])
        log(f"{cfg.name}: traced step (per stage type):\n" + T.format_table(sums[bi]))
        if trace_detail:
            log(f"{cfg.name}: traced step (per stage):\n" + T.format_phases(T.phases(traces[bi], plan)))
        out["trace"] = {"idle_frac": round(sums[bi]["idle_frac"], 4), "step_us": round(sums[bi]["total_us"], 1),
                        "by_type_us": {k: round(v["span_us"], 1) for k, v in T.by_type(sums[bi]).items()}}
    return out


def batch_points(eng, cfg, batches, reps: int = 20):
    """Weight products of one DeepSeek-V3 MoE layer for B tokens at once
    (pdm_batch_gemm on [W_DQ ; W_DKV], W_UQ and W_O, pdm_batch_ffn on the
    union of the B tokens' routed experts plus the shared one), timed with HIP
    events on the launch stream over `reps` back-to-back passes. W_UK / W_UV
    (per-head products, about 1% of the layer's bytes), the bf16 router and
    attention are not in it. Bytes are the FP8 codes and scales of every matrix
    a pass reads; the union is counted from the seeded routing."""
    import torch
    from persistent_decode_megakernel_amd import _lib as L, pack, roofline as R
    from synth import gen
    layer = cfg.layers.index("moe")

    def mat_bytes(name, expert=-1):
        m = pack.packed_layout(cfg, name, layer, expert)
        return m.rows * m.K + (m.rows // 8) * m.n_kblocks * 2

    mats = [("wq_a", cfg.hidden), ("wq_b", cfg.q_lora), ("wo", cfg.n_heads * cfg.v_head)]
    dense_bytes = sum(mat_bytes(n) for n, _ in mats)
    expert_bytes = mat_bytes("w_gate", 0) + mat_bytes("w_down", 0)
    stream = torch.cuda.current_stream()
    pts = []
    for B in batches:
        xs = {n: torch.from_numpy(gen.batch_rows(B, K, SEED, tag=L.TENSOR_IDS[n])).cuda() for n, K in mats}
        ys = {n: torch.empty(B, pack.packed_layout(cfg, n, layer).rows, device="cuda") for n, _ in mats}
        h = torch.from_numpy(gen.batch_rows(B, cfg.hidden, SEED, tag=99)).cuda()
        idx, w = gen.batch_routing(cfg, B, SEED)
        idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
        yf = torch.empty(B, cfg.hidden, device="cuda")
        n_u = len(set(idx.ravel().tolist())) + cfg.n_shared

        def gemms():
            for n, _ in mats:
                eng.batch_gemm(L.TENSOR_IDS[n], layer, xs[n], out=ys[n])

        def ffn():
            eng.batch_ffn(layer, h, idx_d, w_d, out=yf)

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / reps

        t_g, t_f = timed(gemms), timed(ffn)
        t = timed(lambda: (gemms(), ffn()))
        nbytes = dense_bytes + n_u * expert_bytes
        pts.append({"B": B, "us_per_layer_pass": round(t * 1e6, 1), "us_gemms": round(t_g * 1e6, 1),
                    "us_ffn": round(t_f * 1e6, 1), "experts_read": n_u, "weight_bytes": int(nbytes),
                    "GBps": round(nbytes / t / 1e9, 1), "frac_of_8TBps": round(nbytes / t / R.HBM_PEAK_BYTES_PER_S, 4),
                    "tokens_per_s_per_layer": round(B / t, 1), "bytes_per_token": int(nbytes / B)})
        log(f"batch {B}: one MoE layer's weight products {t * 1e6:.1f} us ({n_u} experts, "
            f"{nbytes / 1e6:.0f} MB, {nbytes / t / 1e9:.0f} GB/s); qkv+q_b+W_O {t_g * 1e6:.1f} us, FFN {t_f * 1e6:.1f} us")
    return {"workload": f"{cfg.name} layer {layer}: FP8 weight products of one MoE layer for B tokens "
                        "([W_DQ ; W_DKV], W_UQ, W_O, union-of-experts SwiGLU), synthetic uniform top-8 routing",
            "kernel": "pdm::batch_gemm_kernel (MFMA 16x16x32 bf16, FP8 weights read in place)",
            "points": pts}


def batch_step_points(eng, cfg, batches, steps: int = 16, warm: int = 2):
    """Whole decode steps of B sequences at once on the stack
    (pdm_batch_decode_step): each sequence has its own cache holding the
    workload's prompt latents and steps through teacher-forced random tokens
    at positions prompt_len + j. Timed with HIP events over `steps` steps after
    `warm` untimed ones (which also append cache rows). Per-user speed is 1 /
    step time, total throughput B / step time."""
    import torch
    from synth import gen
    P = cfg.prompt_len
    lat = [gen.latent_rows(cfg, l, P, SEED, device="cuda") for l in range(cfg.n_layers)]
    stream = torch.cuda.current_stream()
    pts = []
    for B in batches:
        caches = eng.batch_caches(B)
        for b in range(B):
            for l in range(cfg.n_layers):
                caches[b, l, :P] = lat[l]
        toks = [[gen.decode_token(cfg, j, 0, SEED + 1 + b) for b in range(B)] for j in range(warm + steps)]
        lg = torch.empty(B, cfg.vocab, device="cuda")
        am = torch.empty(B, dtype=torch.int32, device="cuda")

        def step(j):
            rc = eng.batch_decode_step_raw(toks[j], [P + j] * B, caches, logits=lg, argmax=am)
            if rc != 0:
                raise SystemExit(f"batched step failed: {rc}")
        for j in range(warm):
            step(j)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for j in range(warm, warm + steps):
            step(j)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / steps
        pts.append({"B": B, "ms_per_step": round(t * 1e3, 3), "tok_s_user": round(1 / t, 1),
                    "tok_s_total": round(B / t, 1)})
        log(f"batched step B={B}: {t * 1e3:.3f} ms/step, {1 / t:.1f} tok/s/user, {B / t:.1f} tok/s total")
        del caches
        torch.cuda.empty_cache()
    return {"workload": f"{cfg.name}: B sequences per step, each with its own {P}-position prompt cache, "
                        f"teacher-forced random tokens, context {P + warm + 1}..{P + warm + steps}",
            "api": "pdm_batch_decode_step (host-launched kernels; batched MFMA weight products, union of experts)",
            "points": pts}


def layer_steps(name: str, copies: int, steps: int, warm: int = 2):
    """Microseconds per step of one bare DeepSeek-V3-shaped layer (dense or
    MoE, fed an N(0,1) bf16 hidden vector, 1024-position prompt cache).
    Consecutive steps alternate over `copies` engines that hold their own
    copies of the weights, so a step never finds the weights of the step
    before it in the 256 MB MALL (one dense layer streams ~0.6 GB, a MoE layer
    ~0.6 GB of its ~11 GB). Each step is one launch, timed with HIP events on
    the launch stream; the launch gap between steps is included."""
    import torch
    from persistent_decode_megakernel_amd import Engine, roofline as R
    from synth import configs, gen
    cfg = configs.get(name)
    P = cfg.prompt_len
    n = steps + warm
    per_engine = (n + copies - 1) // copies
    engines = []
    for _ in range(copies):
        e = Engine(cfg, max_ctx=P + per_engine, device=0)
        store = gen.LogicalWeights(cfg, SEED, "cuda", cache=False)
        for spec in store.specs():
            e.load_tensor(spec, store.get(spec.name, spec.layer, spec.expert))
        del store
        e.reset()
        e.import_kv(0, 0, gen.latent_rows(cfg, 0, P, SEED, device="cuda"))
        engines.append(e)
    xs = [gen.layer_input(cfg, j, 0, SEED, device="cuda") for j in range(n)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for j in range(n):
        engines[j % copies].decode(P + j // copies, x_in=xs[j])
        ev[j + 1].record(stream)
    torch.cuda.synchronize()
    for e in engines:
        rc, st = e.status()
        if rc != 0:
            raise SystemExit(f"{name}: layer step failed: status {rc} stage {st.stage}")
    us = sorted(ev[j].elapsed_time(ev[j + 1]) * 1e3 for j in range(warm, n))
    mean_us = sum(us) / len(us)
    ctx = P + per_engine // 2
    nbytes = R.bytes_per_token(cfg, ctx)
    del engines
    torch.cuda.empty_cache()
    log(f"{name}: {mean_us:.1f} us per layer-step (p50 {us[len(us) // 2]:.1f}) over {copies} weight copies, "
        f"{nbytes / mean_us / 1e3:.0f} GB/s")
    return {"workload": name, "weight_copies": copies, "steps": steps, "us_per_layer_step": round(mean_us, 2),
            "p50_us": round(us[len(us) // 2], 2), "bytes_per_step": int(nbytes),
            "GBps": round(nbytes / mean_us / 1e3, 1),
            "frac_of_8TBps": round(nbytes / (mean_us * 1e-6) / R.HBM_PEAK_BYTES_PER_S, 4),
            "timing": "one launch per step (launch gap included), steps alternate over the weight copies"}


def dsa_points(contexts, k: int = 2048, reps: int = 20):
    """Sparse (DSA) attention of one DeepSeek-V3-shaped layer at batch 1: the
    indexer (64 heads x 128 over bf16 keys), the top-k of the scores and MLA
    attention of 128 heads over the k chosen rows of the latent cache, timed
    with HIP events on the launch stream, each call and the three together,
    rotating over enough copies of the caches (>= 1 GB) that the last-level
    cache holds none of them. Dense attention over all n rows through the same
    attention kernel is timed beside it. Algorithmic bytes: the indexer reads
    n keys, the top-k n scores, the attention k cache rows (1152 B each)."""
    import torch
    from persistent_decode_megakernel_amd import dsa as G
    from synth import gen
    HI, dI, H, dc, dr = 64, 128, 128, 512, 64
    tau = 1.0 / math.sqrt(192.0)
    stream = torch.cuda.current_stream()
    pts = []
    for n in contexts:
        per = n * (dI + dc + dr) * 2
        copies = max(2, -(-(1 << 30) // per))
        q, w, keys, rows, q_lat, q_pe = gen.dsa_inputs(n, HI, dI, H, dc, dr, seed=SEED, tag=5)
        qd, wd = torch.from_numpy(q).cuda(), torch.from_numpy(w).cuda()
        ql, qp = torch.from_numpy(q_lat).cuda(), torch.from_numpy(q_pe).cuda()
        kc = [keys.cuda() for _ in range(copies)]
        cc = [rows.cuda() for _ in range(copies)]
        sc = torch.empty(n, device="cuda")
        sel = torch.empty(min(k, n), dtype=torch.int32, device="cuda")
        tw = torch.empty(G.topk_work_bytes(n) // 4, dtype=torch.int32, device="cuda")
        allpos = torch.arange(n, dtype=torch.int32, device="cuda")
        work = torch.empty(G.work_bytes(H, dc) // 4, device="cuda")
        o = torch.empty(H, dc, device="cuda")
        it = [0]

        def nxt():
            it[0] = (it[0] + 1) % copies
            return it[0]

        def f_idx():
            G.index_scores(qd, wd, kc[nxt()], out=sc)

        def f_topk():
            G.topk(sc, k, out=sel, work=tw)

        def f_att():
            G.attention(ql, qp, cc[nxt()], sel, tau, work=work, out=o)

        def f_all():
            c = nxt()
            G.index_scores(qd, wd, kc[c], out=sc)
            G.topk(sc, k, out=sel, work=tw)
            G.attention(ql, qp, cc[c], sel, tau, work=work, out=o)

        def f_dense():
            G.attention(ql, qp, cc[nxt()], allpos, tau, work=work, out=o)

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / reps

        f_idx()
        t_i, t_k, t_a, t_all, t_d = timed(f_idx), timed(f_topk), timed(f_att), timed(f_all), timed(f_dense)
        b_i, b_k, b_a = n * dI * 2, n * 4 + min(k, n) * 4, min(k, n) * (dc + dr) * 2
        pt = {"context": n, "k": min(k, n), "cache_copies": copies,
              "indexer_us": round(t_i * 1e6, 2), "indexer_GBps": round(b_i / t_i / 1e9, 1),
              "topk_us": round(t_k * 1e6, 2),
              "attention_us": round(t_a * 1e6, 2), "attention_GBps": round(b_a / t_a / 1e9, 1),
              "sparse_layer_us": round(t_all * 1e6, 2),
              "dense_attention_us": round(t_d * 1e6, 2),
              "algorithmic_bytes": {"indexer": b_i, "topk": b_k, "attention": b_a}}
        log(f"dsa n={n} k={pt['k']}: indexer {pt['indexer_us']} us, top-k {pt['topk_us']} us, attention "
            f"{pt['attention_us']} us, all three {pt['sparse_layer_us']} us; dense attention over all n "
            f"{pt['dense_attention_us']} us")
        pts.append(pt)
        del kc, cc
        torch.cuda.empty_cache()
    return pts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="dsv3_stack_1k")
    ap.add_argument("--also", default="dsv3_stack_8k",
                    help="second workload timed on the same engine ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--trace-detail", action="store_true",
                    help="also print the per-stage phase breakdown of the fastest traced step (stderr)")
    ap.add_argument("--mxfp4", default="dsv3_stack_1k_fp4",
                    help="the same stack with MXFP4 experts, timed on its own engine ('' for none)")
    ap.add_argument("--layers", default="dsv3_dense_layer,dsv3_moe_layer",
                    help="bare single-layer workloads timed after the stack ('' for none)")
    ap.add_argument("--layer-copies", type=int, default=2,
                    help="weight copies the single-layer steps alternate over")
    ap.add_argument("--layer-steps", type=int, default=32)
    ap.add_argument("--batch", default="1,2,4,8",
                    help="batch sizes of the batched weight-product leg on the stack's engine ('' for none)")
    ap.add_argument("--dsa", default="9216,32768,131072",
                    help="cache lengths of the sparse-attention leg, top-2048 ('' for none)")
    ap.add_argument("--resident-only", action="store_true",
                    help="time only resident launches (no single-step launches): for profiler runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy three times (counter calibration for rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this engine runs batch-1 decode on one GPU; multi-GPU runs are not "
                                   "part of it (a sharded path would split GEMV rows, heads, expert rows "
                                   "and the vocabulary over GPUs)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    from persistent_decode_megakernel_amd import Engine, roofline as R
    from synth import configs, gen

    cfgs = [configs.get(args.workload)] + ([configs.get(args.also)] if args.also else [])
    K, Wm = args.steps, args.warmup
    for c in cfgs:
        if K < 1 or max(K, Wm) > c.decode_steps:
            raise SystemExit(f"--steps and --warmup must be within 1..{c.decode_steps}")
    head = cfgs[0]
    # the workloads share weights (same shapes and seeds): one engine sized for the longest context
    max_ctx = max(c.prompt_len + c.decode_steps for c in cfgs)
    eng = Engine(head, max_ctx=max_ctx, device=0, trace=not args.no_trace)
    eng.set_trace(False)
    log(f"buffers: weights {eng.sizes.weight_bytes / 1e9:.2f} GB, kv {eng.sizes.kv_bytes / 1e6:.1f} MB, "
        f"{eng.sizes.n_stages} stages, {eng.sizes.n_workgroups} workgroups, max_ctx {max_ctx}")
    store = gen.LogicalWeights(head, SEED, "cuda", cache=False)
    t0 = time.time()
    for spec in store.specs():
        eng.load_tensor(spec, store.get(spec.name, spec.layer, spec.expert))
    torch.cuda.synchronize()
    log(f"weights generated and packed in {time.time() - t0:.0f} s")
    ceiling = stream_ceiling(eng.weights)
    log(f"streaming-read ceiling (torch sum over 32 GB of the arena): {ceiling / 1e9:.0f} GB/s")

    results = [run_workload(eng, c, K, Wm, not args.no_trace, args.trace_detail and i == 0, args.resident_only)
               for i, c in enumerate(cfgs)]
    batch = batch_points(eng, head, [int(b) for b in args.batch.split(",") if b]) if args.batch else None
    bsteps = (batch_step_points(eng, head, [int(b) for b in args.batch.split(",") if b])
              if args.batch and head.vocab > 0 else None)
    if args.mxfp4:
        # a second engine: the expert matrices are MXFP4 (everything else as above)
        c4 = configs.get(args.mxfp4)
        e4 = Engine(c4, max_ctx=c4.prompt_len + c4.decode_steps, device=0, trace=not args.no_trace)
        e4.set_trace(False)
        s4 = gen.LogicalWeights(c4, SEED, "cuda", cache=False)
        for spec in s4.specs():
            e4.load_tensor(spec, s4.get(spec.name, spec.layer, spec.expert))
        torch.cuda.synchronize()
        log(f"{c4.name}: weights {e4.sizes.weight_bytes / 1e9:.2f} GB (MXFP4 experts)")
        r4 = run_workload(e4, c4, K, Wm, not args.no_trace, False, args.resident_only)
        r4["weights"] = "MXFP4 routed and shared experts (e2m1, e8m0 scale per 32); everything else as the FP8 stack"
        if args.batch and c4.vocab > 0:
            # batched steps over the same MXFP4 experts (B = 1 and the largest B asked for)
            bl = [int(b) for b in args.batch.split(",") if b]
            r4["batch_step_points"] = batch_step_points(e4, c4, sorted({min(bl), max(bl)}))
        results.append(r4)
        del e4, s4
        torch.cuda.empty_cache()
    h = results[0]
    tpot = h["resident"]["ms_per_step"] / 1e3
    bytes_mean = h["bytes_per_token"]
    achieved = bytes_mean / tpot
    traffic = load_traffic(head.name)
    out = {
        "metric": "batch-1 decode tokens/s/user",
        "value": round(1.0 / tpot, 3),
        "unit": "tok/s/user",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(tpot * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{head.name}: {head.layers.count('dense')} dense + {head.layers.count('moe')} MoE MLA "
                         f"layers + bf16 LM head, DeepSeek-V3 shapes, batch 1, {head.prompt_len}-position prompt "
                         f"cache of synthetic N(0,1) bf16 latents, {K} teacher-forced decode steps of seeded "
                         f"random tokens, one resident launch"),
            "weights": "fp8-e4m3 + bf16 128x128 block scales; router and LM head bf16",
            "prompt_cache": "synthetic N(0,1) bf16 latents",
            "prompt_positions": head.prompt_len,
            "context_range": h["context_range"],
            "batch": 1,
            "mode": "resident (one launch for all steps)",
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(achieved / R.HBM_PEAK_BYTES_PER_S, 4),
                     # per launch like achieved: one resident launch runs all K steps
                     "traffic": None if traffic is None else round(traffic * K),
                     "kernel": "pdm::engine_kernel (one resident launch of all K steps)",
                     "algorithmic_bytes_per_launch": int(bytes_mean * K),
                     "algorithmic_bytes_per_step": int(bytes_mean),
                     "traffic_per_step": traffic,
                     "frac_of_stream_ceiling": round(achieved / ceiling, 4)},
        "stream_ceiling_GBps": round(ceiling / 1e9, 1),
        "workloads": results,
        "seed": SEED,
        "git_head": git_head(),
        "engine_source_hash": engine_source_hash(),
    }
    if batch is not None:
        out["batch_points"] = batch
    if bsteps is not None:
        out["batch_step_points"] = bsteps
    if args.dsa:
        out["dsa_points"] = dsa_points([int(n) for n in args.dsa.split(",") if n])
    if args.layers:
        del eng
        torch.cuda.empty_cache()
        out["layer_steps"] = [layer_steps(n, args.layer_copies, args.layer_steps)
                              for n in args.layers.split(",") if n]
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(head, store, head.prompt_len)
        except Exception as exc:  # the baseline is reported, never required
            out["cpu_baseline"] = {"error": repr(exc)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
