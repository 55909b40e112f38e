#!/usr/bin/env python3
"""Benchmark: MLA decode with weight absorption on one MI355X.

One step = one call of mla_decode over a batch of 32 sequences (absorbed query
projection, split-K flash-decode over the latent cache, split combine and
W_UV projection), one query token per sequence, DeepSeek-V3 shapes (H=128,
d_c=512, d_hR=64, d_nope=128, d_v=128), bf16 cache, cached lengths drawn
uniform in [4096, 8192]. Inputs are synthetic and seeded (mla_synth) and
resident in HBM before timing; each step reads a different copy of the cache
and weights so that no step is served from the 256 MB Infinity Cache.

Prints one JSON line. value = latent-cache bytes read per step / step time
(GB/s), timed over exactly `--steps` steps as a caller runs them (the same
region repeated ten more times gives the p10/p50/p90 of the step time).
The same steps then run once more with the library's per-kernel profiling on
(each kernel starts on an idle stream and records its own start and end):
those give the per-kernel durations and the roofline object, which reports
the split-K kernel alone. The other workloads (uniform 8K batch, one 4K
sequence, 4 x 128K, 128 sequences with fp8 latents and a fused append, and
the ragged batch with 4 query tokens per sequence) are measured the same way
and reported under "workloads".
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
FP16_PEAK_FLOPS = 2.5e15  # MI355X dense fp16 / bf16 matrix cores, published
METRIC = "MLA decode latent-cache read GB/s (% of HBM peak) + tokens/s, B=32 ctx=8K"
DEFAULT_WORKLOAD = "v3_b32_ragged"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "splitk_decode_bf16_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # 300 steps (about 30 ms): the shader clock needs that long to settle
    # after the idle host-side set-up; with 10 the first timed region read
    # 17 % slower than the same steps a moment later
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    p.add_argument("--headline-only", action="store_true",
                   help="time only the headline workload (the others are measured by default)")
    p.add_argument("--calib-mib", type=int, default=0,
                   help="first run one plain device copy of this many MiB (mla_calib_copy), a kernel of known "
                        "traffic for scaling hardware byte counters")
    return p.parse_args()


def kernel_source_hash():
    """Hash of the sources that decide the split-K kernels' traffic: the
    kernels, their headers and the planner (which items they run)."""
    h = hashlib.sha256()
    for f in ("k_splitk.hip", "k_splitk8.hip", "splitk_common.hpp", "device_util.hpp", "mla_internal.hpp",
              "splitk_addr.hpp", "plan_hash.hpp", "mla_api.cpp"):
        with open(os.path.join(ROOT, "compressed_kv_cache_absorbed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_alg):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current split-K source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


DT = {"f32": 0, "bf16": 1, "fp8": 2}


def run_workload(m, torch, name, steps, warmup, q_len=1, repeats=10):
    """Times `steps` decode steps of one workload (after `warmup` untimed ones).
    A step is one mla_decode call, or one mla_append_decode call for the
    workload that appends a token per sequence; that step also restores
    seq_len first (a 4-byte-per-sequence device copy) so every step appends
    at the same place. With q_len > 1 a step is one mla_decode_multi call:
    q_len new query tokens per sequence (the last q_len cached rows)."""
    import mla_synth
    from mla_synth.device import upload

    case = mla_synth.workload(name)
    dev = torch.device("cuda", 0)
    t = upload(case, dev)
    d = m.dims(case.H, case.d_c, case.d_rope, case.d_nope, case.d_v, case.d_model, case.softmax_scale,
               case.rope_base)
    lens = case.lens + case.n_new
    cache_bytes = int(lens.sum()) * case.row_bytes
    weight_bytes = 2 * case.H * case.d_c * case.d_nope * 2
    # enough copies that a step's inputs were last touched >= 768 MB of traffic ago
    ncopy = max(2, math.ceil(768e6 / (cache_bytes + weight_bytes)) + 1)

    def copies(x):
        return None if x is None else [x] + [x.clone() for _ in range(ncopy - 1)]

    rows, scale, wuk, wuv = copies(t["rows"]), copies(t["scale"]), copies(t["w_uk"]), copies(t["w_uv"])
    lat, rope = DT[case.latent_dtype], DT[case.rope_dtype]
    caches = [m.cache(rows[j], case.row_stride, lat, rope, t["seq_start"], t["seq_cap"], t["seq_len"],
                      None if scale is None else scale[j]) for j in range(ncopy)]
    plan = m.mla_plan_create(d, lens.tolist(), 0) if q_len == 1 else m.mla_plan_create_multi(d, lens.tolist(), q_len)
    nbytes = m.mla_decode_workspace_bytes(d, plan)
    if q_len > 1:
        qn, qr = mla_synth.multi_queries(case, q_len, seed=17)
        qn = torch.from_numpy(qn.view(np.int16)).to(dev)
        qr = torch.from_numpy(qr.view(np.int16)).to(dev)
        nbytes = m.mla_decode_multi_workspace_bytes(d, plan, q_len)
    if case.n_new:
        nbytes = max(nbytes, m.mla_append_workspace_bytes(d, case.B, case.n_new))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    m.mla_workspace_init(ws)
    o = torch.empty((case.B, q_len, case.H, case.d_v) if q_len > 1 else (case.B, case.H, case.d_v),
                    dtype=torch.bfloat16, device=dev)
    len0 = t["seq_len"].clone()
    act = DT[case.act_dtype]

    def step(k):
        j = k % ncopy
        if case.n_new:
            t["seq_len"].copy_(len0)
            m.mla_append_decode(d, caches[j], plan, t["h"], case.n_new, t["w_dkv"], t["w_kr"], t["q_nope"],
                                t["q_rope"], None, wuk[j], wuv[j], act, o, 1, ws)
        elif q_len > 1:
            m.mla_decode_multi(d, caches[j], plan, q_len, qn, qr, None, wuk[j], wuv[j], act, o, 1, ws)
        else:
            m.mla_decode(d, caches[j], plan, t["q_nope"], t["q_rope"], None, wuk[j], wuv[j], act, o, 1, ws)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    assert m.mla_device_error(ws) == 0
    # timed region 1: the steps as a caller runs them, nothing else in the
    # stream (this gives `value`)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    # the spread: the same region repeated (an event pair around every step
    # would cost more than the spread itself: each timed event record adds
    # about 14 us to a step here); step_ms holds the per-step time of each
    # repeat
    step_ms = []
    for _ in range(repeats):
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for k in range(steps):
            step(k)
        torch.cuda.synchronize()
        step_ms.append((time.perf_counter() - r0) * 1e3 / steps)
    # timed region 2: the same steps with the library's per-kernel profiling
    # (each kernel starts on an idle stream and records its own start and end)
    per_kernel = {}
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(steps):
        m.mla_prof_begin(max_records=16)
        step(k)
        for name, (ms, n) in m.mla_prof_end().items():
            per_kernel.setdefault(name, []).append(ms / n)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    assert m.mla_device_error(ws) == 0
    ms_step_profiled = (t3 - t2) * 1e3 / steps
    kname = "decode_fp8" if case.latent_dtype == "fp8" else "decode_bf16"
    return dict(case=case, t=t, o=o, d=d, plan=plan, cache_bytes=cache_bytes, ms_step=ms_step, step_ms=step_ms,
                ms_step_profiled=ms_step_profiled, splitk=per_kernel[kname], splitk_ms=float(np.mean(per_kernel[kname])),
                splitk_name=kname, per_kernel=per_kernel, n_items=plan.n_items, ncopy=ncopy, q_len=q_len)


def run_merged(m, torch, steps, warmup, d_x=1536, d_out=7168, repeats=10):
    """Decode from precomputed absorbed weights (mla_decode_merged) on the
    headline workload: x is a 1536-wide query latent, y the 7168-wide layer
    output. The merges run once before timing. A step reads the cache, the
    merged query weight [128, 512, 1536] and the merged output weight
    [7168, 128 x 512] (bf16); the weights alone are far larger than the
    on-package cache, so nothing of the previous step survives in it."""
    import mla_synth
    from mla_synth.device import _t, upload

    case = mla_synth.workload(DEFAULT_WORKLOAD)
    dev = torch.device("cuda", 0)
    t = upload(case, dev)
    d = m.dims(case.H, case.d_c, case.d_rope, case.d_nope, case.d_v, 0, case.softmax_scale, case.rope_base)
    x, w_q, w_o = mla_synth.merged_inputs(case, d_x, d_out, seed=230)
    tx, tq, to = _t(x, dev), _t(w_q, dev), _t(w_o, dev)
    a = torch.empty((case.H, case.d_c, d_x), dtype=torch.bfloat16, device=dev)
    bm = torch.empty((d_out, case.H * case.d_c), dtype=torch.bfloat16, device=dev)
    m.mla_merge_query_weight(d, d_x, tq, t["w_uk"], DT["bf16"], a)
    m.mla_merge_output_weight(d, d_out, to, t["w_uv"], DT["bf16"], bm)
    torch.cuda.synchronize()
    del tq, to
    c = m.cache(t["rows"], case.row_stride, DT[case.latent_dtype], DT[case.rope_dtype], t["seq_start"], t["seq_cap"],
                t["seq_len"], None)
    plan = m.mla_plan_create(d, case.lens.tolist(), 0)
    ws = torch.empty(m.mla_decode_merged_workspace_bytes(d, plan, d_out), dtype=torch.uint8, device=dev)
    m.mla_workspace_init(ws)
    y = torch.empty((case.B, d_out), dtype=torch.bfloat16, device=dev)

    def step():
        m.mla_decode_merged(d, c, plan, d_x, tx, t["q_rope"], None, a, d_out, bm, DT["bf16"], y, DT["bf16"], ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert m.mla_device_error(ws) == 0
    step_ms = []
    for _ in range(repeats + 1):
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        step_ms.append((time.perf_counter() - r0) * 1e3 / steps)
    per_kernel = {}
    for _ in range(steps):
        m.mla_prof_begin(max_records=16)
        step()
        for name, (ms, n) in m.mla_prof_end().items():
            per_kernel.setdefault(name, []).append(ms / n)
    torch.cuda.synchronize()
    assert m.mla_device_error(ws) == 0
    cache_bytes = int(case.lens.sum()) * case.row_bytes
    a_bytes, bm_bytes = a.numel() * 2, bm.numel() * 2
    ms = step_ms[0]
    med = {k: float(np.median(v)) for k, v in per_kernel.items()}
    unmerged = 2 * (case.H * case.d_nope * d_x + 2 * case.H * case.d_nope * case.d_c + d_out * case.H * case.d_v)
    return {"batch": case.B, "d_x": d_x, "d_out": d_out, "cache_bytes_per_step": cache_bytes,
            "merged_weight_bytes": a_bytes + bm_bytes, "unmerged_weight_bytes_w_q_w_uk_w_uv_w_o": unmerged,
            "ms_per_step": round(ms, 5), "step_ms": pct(step_ms[1:]),
            "tokens_per_s": round(case.B / (ms * 1e-3), 1),
            "GBs_step_all_bytes": round((cache_bytes + a_bytes + bm_bytes) / (ms * 1e-3) / 1e9, 2),
            "kernel_ms_p50": {k: round(v, 5) for k, v in med.items()},
            "absorb_merged_GBs": round(a_bytes / (med["absorb_merged"] * 1e-3) / 1e9, 2),
            "out_merged_GBs": round(bm_bytes / (med["out_merged"] * 1e-3) / 1e9, 2),
            "out_merged_hbm_frac": round(bm_bytes / (med["out_merged"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def pct(xs):
    """p10 / p50 / p90 of a list of times (ms), rounded."""
    q = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(q[0]), 5), "p50": round(float(q[1]), 5), "p90": round(float(q[2]), 5)}


def workload_summary(res):
    """One workload: step time (mean and spread), rates against the HBM and
    fp16 matrix-core peaks for the split-K kernel, per-kernel medians."""
    case, ql = res["case"], res["q_len"]
    flops = 2.0 * case.H * ql * (2 * case.d_c + case.d_rope) * float((case.lens + case.n_new).sum())
    sk = res["splitk_ms"]
    return {"batch": case.B, "query_tokens_per_seq": ql, "cache_tokens": int((case.lens + case.n_new).sum()),
            "latent_dtype": case.latent_dtype, "appends": int(case.n_new), "split_items": res["n_items"],
            "cache_bytes_per_step": res["cache_bytes"],
            "ms_per_step": round(res["ms_step"], 5), "step_ms": pct(res["step_ms"]),
            "tokens_per_s": round(case.B * ql / (res["ms_step"] * 1e-3), 1),
            "cache_GBs_step": round(res["cache_bytes"] / (res["ms_step"] * 1e-3) / 1e9, 2),
            "splitk_ms_mean": round(sk, 5), "splitk_ms": pct(res["splitk"]),
            "splitk_GBs": round(res["cache_bytes"] / (sk * 1e-3) / 1e9, 2),
            "splitk_hbm_frac": round(res["cache_bytes"] / (sk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "splitk_mfma_frac_fp16": round(flops / (sk * 1e-3) / FP16_PEAK_FLOPS, 4),
            "step_over_splitk": round(res["ms_step"] / sk, 3),
            "kernel_ms_p50": {k: round(float(np.median(v)), 5) for k, v in res["per_kernel"].items()}}


def cpu_baseline(res, budget_s):
    """The oracle's non-absorbed fp64 decode timed on the host on a bounded
    sample of (sequence, head) pairs, scaled to the whole step; its outputs
    double as a sampled parity check of the last timed step."""
    import numpy as np
    from oracle import mla as omla
    from tests.helpers import act_to_f64, oracle_cache
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info] + [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '')}".strip()
    except Exception:
        cores = os.cpu_count()
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    case = res["case"]
    rng = np.random.default_rng(11)
    seqs = sorted(set(int(x) for x in rng.choice(case.B, size=min(4, case.B), replace=False)))
    C, R = oracle_cache(case, seqs=seqs)
    args = dict(q_nope=act_to_f64(case.q_nope, "bf16"), q_rope=act_to_f64(case.q_rope, "bf16"),
                w_uk=act_to_f64(case.w_uk, "bf16"), w_uv=act_to_f64(case.w_uv, "bf16"))
    done, elapsed, tokens = 0, 0.0, 0
    got, ref = [], []
    o = res["o"].float().cpu().numpy()
    while elapsed < budget_s or done < 4:
        b = seqs[done % len(seqs)]
        i = int(rng.integers(case.H))
        t0 = time.perf_counter()
        r = omla.decode(C, R, case.seq_start, case.lens, args["q_nope"], args["q_rope"], args["w_uk"],
                        args["w_uv"], case.softmax_scale, case.rope_base, pairs=[(b, i)])
        elapsed += time.perf_counter() - t0
        ref.append(r[0])
        got.append(o[b, i])
        tokens += int(case.lens[b])
        done += 1
        if done >= 4000:
            break
    # the same oracle outputs against the last timed step's (bf16) outputs
    got, ref = np.stack(got), np.stack(ref)
    parity = float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))
    # per (token, head) cost, scaled to the step's tokens x heads
    per_tok_head = elapsed / tokens
    step_s = per_tok_head * float(case.lens.sum()) * case.H
    # informational: the oracle's absorbed fp64 form (every head of a sampled
    # sequence at once), scaled the same way
    abs_elapsed, abs_tokens = 0.0, 0
    for b in seqs:
        s0, L = int(case.seq_start[b]), int(case.lens[b])
        t0 = time.perf_counter()
        omla.decode_absorbed_heads(C[s0:s0 + L], R[s0:s0 + L], args["q_nope"][b], args["q_rope"][b], args["w_uk"],
                                   args["w_uv"], case.softmax_scale, case.rope_base, L - 1)
        abs_elapsed += time.perf_counter() - t0
        abs_tokens += L
    abs_step_s = abs_elapsed / abs_tokens * float(case.lens.sum())
    return {"value": round(res["cache_bytes"] / step_s / 1e9, 6), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "step_seconds": round(step_s, 3), "tokens_per_s": round(case.B / step_s, 4),
            "absorbed_value": round(res["cache_bytes"] / abs_step_s / 1e9, 4),
            "absorbed_step_seconds": round(abs_step_s, 4), "cpu_model": cpu_model,
            "host_cpus": os.cpu_count(), "blas": blas, "parity_max_err_over_rms": round(parity, 6),
            "sample": f"{done} (sequence, head) pairs of the workload ({tokens} token-heads, "
                      f"{elapsed:.1f} s of fp64 non-absorbed decode), scaled to {case.B} sequences x {case.H} heads; "
                      f"absorbed_*: the oracle's absorbed fp64 form on all heads of {len(seqs)} sequences "
                      f"({abs_elapsed:.2f} s), informational"}


def stream_read_ceiling(m, torch, mib=4096, reps=20):
    """Achievable HBM read rate: mla_calib_read over a buffer sixteen times
    the 256 MB on-package cache, best of `reps` launches timed with events on
    the launch stream."""
    nb = mib << 20
    src = torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        m.mla_calib_read(src, nb, sink)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        m.mla_calib_read(src, nb, sink)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, sink
    torch.cuda.empty_cache()
    return nb / (best * 1e-3) / 1e9


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the decode path is built and "
              f"measured on a single MI355X, and multi-GPU sharding is design-only.", file=sys.stderr)
        sys.exit(2)
    import torch
    import compressed_kv_cache_absorbed_amd as m
    m.load()
    torch.cuda.set_device(0)
    if a.calib_mib > 0:
        nb = a.calib_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        m.mla_calib_copy(dst, src, nb)
        torch.cuda.synchronize()
        del src, dst
    ceiling = stream_read_ceiling(m, torch)
    res = run_workload(m, torch, a.workload, a.steps, a.warmup)
    case = res["case"]
    gbs = res["cache_bytes"] / (res["ms_step"] * 1e-3) / 1e9
    ach = res["cache_bytes"] / (res["splitk_ms"] * 1e-3) / 1e9
    traffic = measured_traffic(res["cache_bytes"])
    head = workload_summary(res)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(res["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{a.workload}: batch {case.B}, one query token each, H={case.H}, d_c={case.d_c}, "
                               f"d_hR={case.d_rope}, d_nope={case.d_nope}, d_v={case.d_v}, bf16 latent cache, "
                               f"cached lengths U[4096, 8192] (sum {int(case.lens.sum())})",
                   "global_batch": case.B, "cache_bytes_per_step": res["cache_bytes"],
                   "split_items": res["n_items"], "input_copies_rotated": res["ncopy"]},
        "tokens_per_s": round(case.B / (res["ms_step"] * 1e-3), 1),
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "step_ms": head["step_ms"],
        "step_over_splitk": head["step_over_splitk"],
        "kernel_ms_p50": head["kernel_ms_p50"],
        "ms_per_step_profiled": round(res["ms_step_profiled"], 5),
        "roofline": {"kernel": "splitk_decode (bf16 latent)", "bound": "hbm", "achieved": round(ach, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "per_launch_bytes": res["cache_bytes"], "avg_launch_ms": round(res["splitk_ms"], 5),
                     "launch_ms": head["splitk_ms"], "mfma_frac_fp16": head["splitk_mfma_frac_fp16"],
                     "stream_read_GBs": round(ceiling, 1), "frac_of_stream_read": round(ach / ceiling, 4)},
    }
    if not a.headline_only:
        out["workloads"] = {}
        for name, ql in (("v3_b32_8k", 1), ("v3_b1_4k", 1), ("v3_b4_128k", 1), ("v3_b128_fp8", 1),
                         ("v3_b32_ragged", 4)):
            r = run_workload(m, torch, name, a.steps, a.warmup, q_len=ql)
            out["workloads"][name if ql == 1 else f"{name}_{ql}_query_tokens"] = workload_summary(r)
            print(f"# {name} q_len {ql}: {out['workloads'][name if ql == 1 else f'{name}_{ql}_query_tokens']['ms_per_step']} ms/step",
                  file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()
        out["workloads"]["v3_b32_ragged_merged_weights"] = run_merged(m, torch, a.steps, a.warmup)
        print(f"# merged weights: {out['workloads']['v3_b32_ragged_merged_weights']['ms_per_step']} ms/step",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(res, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
