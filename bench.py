#!/usr/bin/env python3
"""bs=1 decode throughput of the llama-8B-shaped decoder on one MI355X.

One step is one decode token through the whole step list (embed, 32 layers
of rms_norm / q,k,v matmul / rope / attention over the KV cache / o matmul /
add / rms_norm / gate,up matmul / silu / mul / down matmul / add, final
rms_norm, logits matmul) plus the greedy argmax, at context 4096 onwards.
The context is built by one bulk prefill of a 4096-token synthetic prompt,
timed and reported as prefill tokens/s. Weights are random with the shape's
distributions (f16 matmul weights ~N(0, 0.02), norms ~1+N(0, 0.02)), drawn
on the GPU from a seeded generator; token ids are synthetic.

Prints one JSON line (see the keys in `report`):
  value          decode tokens/s over the timed steps
  roofline       the gate/up matvec (the largest kernel: 47% of a step's
                 bytes): algorithmic bytes per launch / mean launch time,
                 the step's launches replayed back to back between HIP
                 events on the library's stream, vs 8 TB/s
  cpu_baseline   the CPU oracle on a bounded sample of the same step
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "bs=1 decode tokens/s (8B shape, ctx 4096); achieved HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg: dict, p: int) -> int:
    """Algorithmic HBM bytes of one decode step at position p: every matmul
    weight once (f16, or 8-bit values + f16 scales), the norm weights and
    biases as held on the device (f32), one embedding row, the KV rows 0..p-1
    (within the window on a sliding-window layer) read and row p written
    (f32), and the logits written."""
    d, F, V, L = cfg["d_model"], cfg["ffn_dim"], cfg["vocab"], cfg["n_layers"]
    hd = cfg["head_dim"]
    qd, kvd = cfg["n_heads"] * hd, cfg["n_kv_heads"] * hd
    per_layer = (qd + 2 * kvd) * d + d * qd + 2 * F * d + d * F
    mat = L * per_layer + V * d  # lm head (untied)
    wbytes = mat * 2 if cfg["wdtype"] == "f16" else mat + mat // 32 * 2
    norms = (L * 2 * d + d) * 4
    if cfg["arch"] in ("qwen3", "gemma3"):
        norms += L * 2 * hd * 4
    if cfg["arch"] == "gemma3":  # rms_norm weights of the o and down outputs
        norms += L * 2 * d * 4
    if cfg["arch"] == "qwen2":  # q/k/v biases, f32 on the device
        norms += L * (qd + 2 * kvd) * 4
    # KV rows read: positions 0..p, or the last `sliding_window` of them on a
    # local layer
    W, P = cfg.get("sliding_window", 0), cfg.get("window_pattern", 1)
    rows = sum(min(p + 1, W) if W and (i + 1) % P else p + 1 for i in range(L))
    return wbytes + norms + d * 2 + rows * 2 * kvd * 4 + V * 4


def gate_up_launch_bytes(cfg: dict) -> int:
    """One gate/up launch: per output unit a gate row and an up row of d
    weights (16,384 bytes in f16 at d = 4096), times ffn_dim units, plus the
    activation and norm weight read once and the ffn_dim outputs written."""
    d, F = cfg["d_model"], cfg["ffn_dim"]
    unit = 2 * d * (2 if cfg["wdtype"] == "f16" else 1)
    if cfg["wdtype"] == "q8":
        unit += 2 * (d // 32) * 2
    return F * unit + d * 4 + d * 4 + F * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_matvec_llama8b_traffic.txt")
TRAFFIC_SOURCES = [os.path.join(ROOT, "decoder_forward_amd", "csrc", f)
                   for f in ("device_common.h", "decode.hip", "kernels.h")]


def kernel_source_hash() -> str:
    """sha1 of the sources the decode matvec is compiled from."""
    import hashlib
    h = hashlib.sha1()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic() -> dict | None:
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    same counter reads for a plain copy of known size), or None when that
    summary is missing or was taken on other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("source_sha1") != kernel_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_launch"]) * float(kv["copy_fetch_factor"]) * 1024
        write = float(kv["write_kib_per_launch"]) * float(kv["copy_write_factor"]) * 1024
        return {"fetch": fetch, "write": write}
    except (OSError, KeyError, ValueError):
        return None


# MI355X: GRBM_GUI_ACTIVE counts cycles on each of the 8 XCDs (summed);
# SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of the 1024 SIMDs.
N_XCD, N_SIMD = 8, 1024


def pmc_summary(path: str, pattern: str, us_range=None) -> None:
    """Mean of each counter per dispatch over the kernels whose name contains
    `pattern` (and, with us_range, whose duration lies in [lo, hi] us), from
    a rocprofv3 --pmc csv output directory, with the mean dispatch duration
    and, where the counters are there, the clock (GRBM_GUI_ACTIVE per XCD over
    the duration), the fraction of cycles the matrix cores are busy, and the
    LDS bank-conflict share of LDS-active cycles."""
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    disp: dict = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if pattern in r["Kernel_Name"]:
                d = disp.setdefault((f, r["Dispatch_Id"]), {
                    "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
    if us_range:
        lo, hi = us_range
        disp = {k: d for k, d in disp.items() if lo <= d["us"] <= hi}
    if not disp:
        print("no dispatches")
        return
    acc: dict = {}
    for d in disp.values():
        for k, v in d.items():
            acc.setdefault(k, []).append(v)
    mean = {k: sum(v) / len(v) for k, v in acc.items()}
    for k, v in sorted(acc.items()):
        if k != "us":
            print(f"{k}: dispatches {len(v)}, mean {mean[k]:.1f}, min {min(v):.1f}, max {max(v):.1f}")
    us = mean["us"]
    print(f"duration: dispatches {len(acc['us'])}, mean {us:.2f} us, min {min(acc['us']):.2f}, "
          f"max {max(acc['us']):.2f}")
    gui = mean.get("GRBM_GUI_ACTIVE")
    if gui:
        cyc = gui / N_XCD
        print(f"clock: {cyc / us / 1e3:.2f} GHz (GRBM_GUI_ACTIVE / {N_XCD} XCDs / duration)")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            print(f"MFMA busy: {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * N_SIMD):.3f} of the cycles of "
                  f"{N_SIMD} SIMDs")
    if mean.get("SQ_LDS_IDX_ACTIVE"):
        print(f"LDS bank conflicts: {mean.get('SQ_LDS_BANK_CONFLICT', 0.0) / mean['SQ_LDS_IDX_ACTIVE']:.3f} "
              f"of LDS-active cycles")


def copy_probe(mib: int) -> None:
    """A plain device copy of `mib` MiB, 4 times (the reference kernel for
    scaling the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy probe: {mib} MiB x 4", flush=True)


def cpu_baseline(cfg: dict, ctx: int) -> dict:
    """The oracle, as it is, on a bounded sample of one decode step: a model
    with the same shapes but 2 of the 32 layers (plus embed and the logits
    matmul), the KV cache restored to `ctx` synthetic positions; the step time
    is scaled to the full layer count with the 0-layer time subtracted."""
    import numpy as np
    import oracle
    import synth
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    c2 = dict(cfg, n_layers=2, max_ctx=ctx + 4)
    W = synth.make_weights(c2)
    m2 = oracle.Model(c2, W)
    for layer in range(2):
        K, V = synth.make_kv_rows(c2, layer, ctx)
        m2.kv_write(layer, 0, 0, K)
        m2.kv_write(layer, 1, 0, V)
    c0 = dict(c2, n_layers=0)
    m0 = oracle.Model(c0, W)
    tok = int(synth.make_prompt(cfg, 1, stream=7)[0])

    def time_one(m, reps):
        ts = []
        for _ in range(reps):
            m.set_kv_len(ctx if m is m2 else 0)
            t = time.perf_counter()
            m.forward([tok])
            ts.append(time.perf_counter() - t)
        return min(ts)
    time_one(m2, 1)
    t2 = time_one(m2, 4)
    t0 = time_one(m0, 4)
    per_layer = max(0.0, (t2 - t0) / 2)
    t_tok = t0 + cfg["n_layers"] * per_layer
    m2.close()
    m0.close()
    try:
        cpu = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
               if l.startswith("model name")][0]
    except Exception:
        cpu = "unknown"
    return {"value": round(1.0 / t_tok, 4), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"one decode step at context {ctx} through 2 of {cfg['n_layers']} "
                       f"layers plus embed and logits (best of 4), 0-layer time "
                       f"{t0 * 1e3:.0f} ms, per-layer {per_layer * 1e3:.0f} ms, "
                       f"scaled to {cfg['n_layers']} layers; cpu {cpu}")}


PEAK_MFMA_F16_TFLOPS = 2500.0


def prefill_classes(dfa, m, cfg, S):
    """Per-layer device time of each bulk-prefill launch class at S rows
    (df_time_prefill: every layer's launches once, back to back between HIP
    events) and the algorithmic flops of its GEMM (2 S N K; the causal
    attention kernel 2 S^2 hd n_heads, QK^T and PV over the lower triangle)
    against the MFMA peak, or for the row pass before the attention (bias /
    norm_heads / rope, KV append, f16 copies of the new rows) its algorithmic
    bytes against HBM; then the MFMA roofline of the dominant class, the
    gate/up GEMM. Runs after decode timing, on an emptied cache (the replays
    write rows 0..S-1)."""
    d, F, hd = cfg["d_model"], cfg["ffn_dim"], cfg["head_dim"]
    qd, kvd = cfg["n_heads"] * hd, cfg["n_kv_heads"] * hd
    flops = {"qkv": 2 * S * (qd + 2 * kvd) * d, "attn": 2 * S * S * hd * cfg["n_heads"],
             "o": 2 * S * d * qd, "gate_up": 2 * S * 2 * F * d, "down": 2 * S * d * F}
    # row pass: read q|k|v f32, write q f16 and the K, V cache rows f32; the
    # f16 copies (head_dim 64 and 128) read the new K, V rows and write them
    # in f16
    rows_bytes = S * (qd + 2 * kvd) * 4 + S * qd * 2 + 2 * S * kvd * 4
    if hd in (64, 128):
        rows_bytes += 2 * S * kvd * 4 + 2 * S * kvd * 2
    out = {}
    for k in ("qkv", "rows", "attn", "o", "gate_up", "down"):
        us = dfa.df_time_prefill(m.h, k, S, reps=1)
        if k == "rows":
            gbps = rows_bytes / (us * 1e-6) / 1e9
            out[k] = {"mean_us_per_layer": round(us, 1), "gbps": round(gbps, 1),
                      "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4), "bytes": rows_bytes}
            continue
        out[k] = {"mean_us_per_layer": round(us, 1), "tflops": round(flops[k] / (us * 1e-6) / 1e12, 1),
                  "mfma_frac": round(flops[k] / (us * 1e-6) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)}
    log(f"[bench] prefill classes at S={S}: {json.dumps(out)}")
    g = out["gate_up"]
    roof = {"bound": "mfma", "kernel": "prefill gate/up GEMM (f16 MFMA, silu * up epilogue)",
            "achieved": g["tflops"], "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": g["mfma_frac"], "flops_per_launch": flops["gate_up"],
            "mean_launch_us": g["mean_us_per_layer"],
            "timing": f"one launch per layer for all {cfg['n_layers']} layers back to back at S={S}, "
                      "HIP events on the library's stream (includes the row rms_norm launch)"}
    return out, roof


def concurrent_sessions(m, cfg, ctx, max_ctx, first, args):
    """N conversations on the model's weights (df_session), each with the
    same restored context, decoding args.steps greedy tokens at once from N
    host threads (one stream each). Aggregate tokens/s over the wall time
    from the common start to the last stream's end."""
    import threading
    import numpy as np
    import torch
    import decoder_forward_amd as dfa
    import synth
    n = args.sessions
    sess = [m.session(max_ctx) for _ in range(n)]
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows_device(cfg, layer, ctx)
        K, V = K.cpu().numpy(), V.cpu().numpy()
        for s in sess:
            s.write_kv(layer, 0, 0, K, ctx)
            s.write_kv(layer, 1, 0, V, ctx)
    outs = [torch.empty(args.steps, dtype=torch.int32, device=m.device) for _ in sess]
    for s, o in zip(sess, outs):  # warm each session's step graph
        dfa.df_generate(s.h, first, 2, o, s.logits)
    torch.cuda.synchronize()
    for s in sess:
        s.write_kv(0, 0, 0, np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"]), np.float32), ctx)
    go = threading.Barrier(n + 1)

    def run(k):
        go.wait()
        dfa.df_generate(sess[k].h, first, args.steps, outs[k], sess[k].logits)
        torch.cuda.synchronize(m.device)

    th = [threading.Thread(target=run, args=(k,)) for k in range(n)]
    for t in th:
        t.start()
    go.wait()
    t0 = time.perf_counter()
    for t in th:
        t.join()
    wall = time.perf_counter() - t0
    same = all(torch.equal(outs[0], o) for o in outs[1:])
    for s in sess:
        s.close()
    agg = n * args.steps / wall
    log(f"[bench] {n} sessions at once: {agg:.1f} tok/s aggregate, "
        f"{wall / args.steps * 1e3:.3f} ms per step each (wall); identical tokens: {same}")
    return {"n": n, "aggregate_tokens_per_s": round(agg, 1),
            "ms_per_step_each": round(wall / args.steps * 1e3, 4),
            "identical_tokens": bool(same),
            "timing": "host wall clock from a common start to the last thread's device sync"}


# The pages' only sizing figure: about 200 MB of activation pool for a 7B
# decoder at bs=1 on their wgpu backend (page "Execution contract", "Memory
# lifecycle", "Activations"). Context for the pool bytes reported here.
PAGES_POOL_BYTES = 200e6


def copy_bandwidth(gib: int = 2) -> dict:
    """Device-to-device copy of `gib` GiB (torch copy_, 8 repetitions between
    events): read + write bytes per second, the achievable streaming rate of
    the box next to the 8 TB/s peak."""
    import torch
    n = gib * (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(8):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / 8
    gbps = 2 * n * 4 / sec / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": round(gbps, 1), "bytes_per_copy": 2 * n * 4,
            "how": f"torch copy_ of {gib} GiB f32 on the device, read + write bytes, mean of 8"}


def cpu_prefill_sample(cfg: dict, S: int) -> dict:
    """The oracle's bulk prefill rate on a bounded sample: the oracle runs a
    bulk call token by token (bulk equals token-by-token inside it), so one
    prompt token at context S/2 (the mean context of an S-token prompt)
    through 2 of the layers, no logits, with the KV cache restored to S/2
    synthetic rows, and through 0 layers; the per-token time is scaled to
    the full layer count and S tokens."""
    import oracle
    import synth
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    mid = S // 2
    c2 = dict(cfg, n_layers=2, max_ctx=mid + 4)
    W = synth.make_weights(c2)
    m2 = oracle.Model(c2, W)
    for layer in range(2):
        K, V = synth.make_kv_rows(c2, layer, mid)
        m2.kv_write(layer, 0, 0, K)
        m2.kv_write(layer, 1, 0, V)
    m0 = oracle.Model(dict(c2, n_layers=0), W)
    tok = int(synth.make_prompt(cfg, 1, stream=7)[0])

    def time_one(m, kv, reps):
        ts = []
        for _ in range(reps):
            m.set_kv_len(kv)
            t = time.perf_counter()
            m.forward([tok], logits=False)
            ts.append(time.perf_counter() - t)
        return min(ts)
    time_one(m2, mid, 1)
    t2, t0 = time_one(m2, mid, 3), time_one(m0, 0, 3)
    per_layer = max(0.0, (t2 - t0) / 2)
    t_tok = t0 + cfg["n_layers"] * per_layer
    m2.close()
    m0.close()
    return {"value": round(1.0 / t_tok, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"one prompt token at context {mid} (the mean context of a {S}-token prompt) "
                       f"through 2 of {cfg['n_layers']} layers without logits (best of 3), "
                       f"0-layer time {t0 * 1e3:.1f} ms, per-layer {per_layer * 1e3:.1f} ms, scaled to "
                       f"{cfg['n_layers']} layers; a {S}-token prefill takes about "
                       f"{S * t_tok:.0f} s")}


def decode_run(dfa, cfg, ctx, steps, warmup, context_from, tag):
    """Load `cfg` (random device weights), build a context of `ctx`
    positions, then time `steps` greedy decode steps (df_generate) between
    HIP events on the model's stream. Returns the open model and the
    figures."""
    import numpy as np
    import torch
    import synth
    max_ctx = ctx + max(steps, warmup) + 8
    log(f"[bench] {tag}: generating weights on the GPU")
    W = synth.make_weights_device(cfg)
    torch.cuda.synchronize()
    m = dfa.Model(cfg, W, max_ctx=max_ctx)
    del W
    torch.cuda.empty_cache()
    first = int(synth.make_prompt(cfg, 1, stream=3)[0])
    # the decode step's own activation pool, before any bulk prefill
    m.forward([first], logits=True)
    torch.cuda.synchronize()
    pool_decode = m.timings()["pool_bytes"]
    m.reset()
    res = {"load_ms": m.timings()["load_ms"], "pool_decode_bytes": pool_decode}
    if context_from == "prefill":
        prompt = synth.make_prompt(cfg, ctx, stream=0)
        m.forward(prompt[:8], logits=False)  # warm the bulk path
        m.reset()
        torch.cuda.synchronize()
        m.forward(prompt, logits=True)
        torch.cuda.synchronize()
        res["prefill_ms"] = m.timings()["last_prefill_ms"]  # HIP events around the launches
        res["prefill_tokens_per_s"] = ctx / (res["prefill_ms"] / 1e3)
        log(f"[bench] {tag}: bulk prefill of {ctx} tokens: {res['prefill_ms']:.1f} ms "
            f"({res['prefill_tokens_per_s']:.0f} tokens/s)")
    else:
        for layer in range(cfg["n_layers"]):
            K, V = synth.make_kv_rows_device(cfg, layer, ctx)
            m.write_kv(layer, 0, 0, K.cpu().numpy(), ctx)
            m.write_kv(layer, 1, 0, V.cpu().numpy(), ctx)
        log(f"[bench] {tag}: restored {ctx} synthetic KV positions")
    assert m.kv_len == ctx
    res["pool_total_bytes"] = m.timings()["pool_bytes"]

    def rewind():  # kv_len back to the context; rows past it are rewritten
        m.write_kv(0, 0, 0, np.zeros((cfg["n_kv_heads"], 0, cfg["head_dim"]), np.float32), ctx)

    if warmup > 0:  # also captures the step graph
        m.generate(first, warmup)
    torch.cuda.synchronize()
    rewind()
    toks = torch.empty(steps, dtype=torch.int32, device=m.device)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(m.stream)
    dfa.df_generate(m.h, first, steps, toks, m.logits)
    ev1.record(m.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = ev0.elapsed_time(ev1)
    total_bytes = sum(step_bytes(cfg, ctx + i) for i in range(steps))
    res.update(value=steps / (dev_ms / 1e3), ms_per_step=dev_ms / steps,
               achieved=total_bytes / (dev_ms / 1e3) / 1e9, wall=wall,
               mean_step_bytes=total_bytes / steps)
    res["hbm_frac"] = res["achieved"] / PEAK_HBM_GBPS
    log(f"[bench] {tag}: decode {steps} steps at {ctx}..: {res['ms_per_step']:.3f} ms/step, "
        f"{res['value']:.1f} tok/s, {res['achieved']:.0f} GB/s ({res['hbm_frac']:.1%} of 8 TB/s); "
        f"wall {wall:.3f} s")
    return m, res


def extra_workloads(dfa, args) -> dict:
    """The other timed configurations, each on its own model: 8-bit blocks at
    contexts 1024 and 8192 (128 steps each), and the qwen3-8B shape's bulk
    prefill of 2048 tokens followed by 64 decode steps."""
    import synth
    out = {}
    cfg = synth.config("llama_8b_q8")
    for ctx in (1024, 8192):
        m, r = decode_run(dfa, cfg, ctx, 128, 8, "prefill", f"llama_8b_q8 ctx {ctx}")
        m.close()
        out[f"llama_8b_q8_ctx{ctx}"] = {
            "decode_tokens_per_s": round(r["value"], 1), "ms_per_step": round(r["ms_per_step"], 4),
            "achieved_hbm_gbps": round(r["achieved"], 1), "hbm_frac": round(r["hbm_frac"], 4),
            "steps": 128, "positions": f"{ctx}..{ctx + 127}",
            "prefill_tokens_per_s": round(r["prefill_tokens_per_s"], 1)}
    cfg = synth.config("qwen3_8b")
    m, r = decode_run(dfa, cfg, 2048, 64, 8, "prefill", "qwen3_8b bulk 2048")
    m.close()
    out["qwen3_8b_bulk2048"] = {
        "prefill_tokens_per_s": round(r["prefill_tokens_per_s"], 1), "prefill_ms": round(r["prefill_ms"], 2),
        "decode_tokens_per_s": round(r["value"], 1), "ms_per_step": round(r["ms_per_step"], 4),
        "hbm_frac": round(r["hbm_frac"], 4), "steps": 64, "positions": "2048..2111"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--context", type=int, default=4096)
    ap.add_argument("--workload", default="llama_8b",
                    choices=["llama_8b", "llama_8b_q8", "qwen3_8b", "qwen3_0p6b", "qwen2_7b",
                             "gemma3_4b"])
    ap.add_argument("--context-from", default="prefill", choices=["prefill", "restore"],
                    help="build the context by bulk prefill of a uniform-random prompt "
                         "(default, timed) or by writing synthetic KV rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 8-bit and qwen3-8B workloads timed after the headline")
    ap.add_argument("--sessions", type=int, default=0, metavar="N",
                    help="also time N conversations (df_session) decoding at once, "
                         "one host thread and stream each, same context")
    ap.add_argument("--copy-probe", type=int, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("DIR", "KERNEL"),
                    help="only summarise a rocprofv3 --pmc output directory")
    ap.add_argument("--pmc-us", nargs=2, type=float, metavar=("LO", "HI"),
                    help="with --pmc-summary: only dispatches lasting LO..HI us")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, us_range=args.pmc_us)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs a model on one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported (sharding a model over "
              f"several GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch
    import decoder_forward_amd as dfa
    import synth
    dfa.lib()  # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    cfg = synth.config(args.workload)
    ctx = args.context
    m, run = decode_run(dfa, cfg, ctx, args.steps, args.warmup, args.context_from, args.workload)
    value, ms_per_step, achieved = run["value"], run["ms_per_step"], run["achieved"]
    prefill_tps = run.get("prefill_tokens_per_s")

    # Per-kernel mean launch time in the same launch configuration: one
    # step's launches of a class replayed back to back between two HIP
    # events on the library's stream (no other work, no per-launch markers).
    kernels = {}
    per_step = {"embed": 1, "logits": 1, "argmax": 1}
    for k in ("qkv", "attn", "attn_merge", "o", "gate_up", "down", "logits", "argmax", "embed"):
        us = dfa.df_time_kernel(m.h, k, reps=8)
        n = per_step.get(k, cfg["n_layers"])
        kernels[k] = {"launches_per_step": n, "mean_us": round(us, 2),
                      "ms_per_step": round(us * n / 1e3, 4)}
    log(f"[bench] kernels: {json.dumps(kernels)}")
    m.reset()  # the prefill replays write cache rows past kv_len: all S of them
    prefill_kernels, pf_roof = prefill_classes(dfa, m, cfg, ctx) if args.context_from == "prefill" else ({}, None)

    gu = kernels["gate_up"]
    traffic = measured_traffic() if args.workload == "llama_8b" else None
    dom = {"kernel": "gate/up matvec (rms_norm + gate,up matmul + silu * up)",
           "bytes": gate_up_launch_bytes(cfg), "us": gu["mean_us"], "traffic": traffic}
    dom_gbps = dom["bytes"] / (dom["us"] * 1e-6) / 1e9

    sessions = concurrent_sessions(m, cfg, ctx, ctx + max(args.steps, args.warmup) + 8, 
                                   int(synth.make_prompt(cfg, 1, stream=3)[0]), args) \
        if args.sessions > 0 else None
    t = m.timings()
    m.close()
    torch.cuda.empty_cache()

    copy = copy_bandwidth()
    log(f"[bench] device copy: {copy['gbps']:.0f} GB/s (read + write)")
    extra = None if args.no_extra else extra_workloads(dfa, args)

    cpu = cpu_pf = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded samples)")
        cpu = cpu_baseline(cfg, ctx)
        log(f"[bench] cpu decode baseline: {cpu}")
        cpu_pf = cpu_prefill_sample(cfg, ctx)
        log(f"[bench] cpu prefill baseline: {cpu_pf}")
        cpu["prefill"] = cpu_pf

    traffic = dom["traffic"]
    report = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.workload}: bs=1 greedy decode, positions {ctx}..{ctx + args.steps - 1}, "
                         f"{cfg['n_layers']} layers, d_model {cfg['d_model']}, "
                         f"{cfg['n_heads']}/{cfg['n_kv_heads']} heads of {cfg['head_dim']}, "
                         f"ffn {cfg['ffn_dim']}, vocab {cfg['vocab']}, "
                         f"{cfg['wdtype']} weights, f32 activations and KV cache"),
            "batch": 1,
            "context": ctx,
            "context_from": args.context_from,
            "weight_dtype": cfg["wdtype"],
            "decode_launch": "one launch per operation class, captured in a HIP graph",
        },
        "achieved_hbm_gbps": round(achieved, 1),
        "hbm_frac": round(achieved / PEAK_HBM_GBPS, 4),
        "copy_bandwidth_gbps": copy["gbps"],
        "hbm_frac_of_copy": round(achieved / copy["gbps"], 4),
        "prefill_tokens_per_s": round(prefill_tps, 1) if prefill_tps else None,
        "roofline": {
            "bound": "hbm",
            "kernel": dom["kernel"],
            "achieved": round(dom_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
            "traffic": round(traffic["fetch"] + traffic["write"]) if traffic else None,
            "traffic_read_write": ([round(traffic["fetch"]), round(traffic["write"])]
                                   if traffic else None),
            "bytes_per_launch": dom["bytes"],
            "mean_launch_us": dom["us"],
            "timing": ("back-to-back replay of one step's launches of the kernel x 8, "
                       "HIP events on the library's stream"),
            "step_frac": round(achieved / PEAK_HBM_GBPS, 4),
        },
        "kernels": kernels,
        "prefill_roofline": pf_roof,
        "prefill_kernels": prefill_kernels,
        "extra_workloads": extra,
        "sessions": sessions,
        "cpu_baseline": cpu,
        "memory": {"weight_bytes": t["weight_bytes"], "kv_bytes": t["kv_bytes"],
                   "activation_pool_bytes": t["pool_bytes"],
                   "activation_pool_decode_bytes": run["pool_decode_bytes"],
                   "activation_pool_prefill_bytes": run["pool_total_bytes"] - run["pool_decode_bytes"],
                   "pages_pool_bytes_context": PAGES_POOL_BYTES,
                   "pages_pool_note": ("the pages' one sizing figure: about 200 MB of activation pool "
                                       "for a 7B decoder at bs=1 on their wgpu backend")},
    }
    print(json.dumps(report), flush=True)


if __name__ == "__main__":
    main()
