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
(GB/s), timed over exactly `--steps` steps as a caller runs them. The same
steps then run once more with an event pair recorded by every kernel dispatch
(hipExtLaunchKernelGGL, on the launch stream): those give the per-kernel
durations and the roofline object, which reports the split-K kernel alone.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "MLA decode latent-cache read GB/s (% of HBM peak) + tokens/s, B=32 ctx=8K"
DEFAULT_WORKLOAD = "v3_b32_ragged"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "splitk_decode_bf16_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    p.add_argument("--extra", action="store_true",
                   help="also time the other workloads (uniform 8K batch, one 4K sequence, 4 x 128K, fp8 + append)")
    p.add_argument("--calib-mib", type=int, default=0,
                   help="first run one plain device copy of this many MiB (mla_calib_copy), a kernel of known "
                        "traffic for scaling hardware byte counters")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("k_splitk.hip", "device_util.hpp", "mla_internal.hpp"):
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


def run_workload(m, torch, name, steps, warmup, q_len=1):
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
    plan = m.mla_plan_create(d, lens.tolist(), 0)
    nbytes = m.mla_decode_workspace_bytes(d, plan)
    if q_len > 1:
        import numpy as np
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
    # timed region 1: the steps as a caller runs them (no profiling events)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    # timed region 2: the same steps again with an event pair recorded by
    # every kernel dispatch (per-kernel durations; the events themselves add
    # some microseconds per dispatch, so region 1 gives the step time)
    m.mla_prof_begin(max_records=8 * steps + 16)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(steps):
        step(k)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    prof = m.mla_prof_end()
    assert m.mla_device_error(ws) == 0
    ms_step_profiled = (t3 - t2) * 1e3 / steps
    kname = "decode_fp8" if case.latent_dtype == "fp8" else "decode_bf16"
    kms, kn = prof[kname]
    splitk_ms = kms / kn
    return dict(case=case, t=t, o=o, d=d, plan=plan, cache_bytes=cache_bytes, ms_step=ms_step,
                ms_step_profiled=ms_step_profiled, splitk_ms=splitk_ms, splitk_name=kname,
                prof={k: v[0] / v[1] for k, v in prof.items()}, n_items=plan.n_items, ncopy=ncopy, q_len=q_len)


def workload_summary(res):
    """One line per extra workload: step and split-K rates, per-kernel times."""
    case, ql = res["case"], res["q_len"]
    flops = 2.0 * case.H * ql * (2 * case.d_c + case.d_rope) * float((case.lens + case.n_new).sum())
    return {"batch": case.B, "query_tokens_per_seq": ql, "cache_tokens": int((case.lens + case.n_new).sum()),
            "latent_dtype": case.latent_dtype, "appends": int(case.n_new),
            "ms_per_step": round(res["ms_step"], 5),
            "tokens_per_s": round(case.B * ql / (res["ms_step"] * 1e-3), 1),
            "cache_GBs_step": round(res["cache_bytes"] / (res["ms_step"] * 1e-3) / 1e9, 2),
            "splitk_GBs": round(res["cache_bytes"] / (res["splitk_ms"] * 1e-3) / 1e9, 2),
            "splitk_hbm_frac": round(res["cache_bytes"] / (res["splitk_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "splitk_mfma_frac_fp16": round(flops / (res["splitk_ms"] * 1e-3) / 2.5e15, 4),
            "kernel_ms": {k: round(v, 5) for k, v in res["prof"].items()}}


def sampled_parity(res, n=8):
    """Sampled outputs of the last step against the oracle (absorbed form,
    pinned equal to the definition): max|err| / rms over the sample."""
    import numpy as np
    from tests.helpers import oracle_cache, oracle_decode
    case = res["case"]
    rng = np.random.default_rng(7)
    pairs = [(int(rng.integers(case.B)), int(rng.integers(case.H))) for _ in range(n)]
    seqs = sorted({b for b, _ in pairs})
    C, R = oracle_cache(case, seqs=seqs)
    ref = oracle_decode(case, pairs=pairs, absorbed=True, C=C, R=R)
    o = res["o"].float().cpu().numpy()
    got = np.stack([o[b, i] for b, i in pairs])
    return float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))


def cpu_baseline(res, budget_s):
    """The oracle's non-absorbed fp64 decode timed on the host on a bounded
    sample of (sequence, head) pairs, scaled to the whole step."""
    import numpy as np
    from oracle import mla as omla
    from tests.helpers import act_to_f64, oracle_cache
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    case = res["case"]
    rng = np.random.default_rng(11)
    seqs = sorted(set(int(x) for x in rng.choice(case.B, size=min(4, case.B), replace=False)))
    C, R = oracle_cache(case, seqs=seqs)
    args = dict(q_nope=act_to_f64(case.q_nope, "bf16"), q_rope=act_to_f64(case.q_rope, "bf16"),
                w_uk=act_to_f64(case.w_uk, "bf16"), w_uv=act_to_f64(case.w_uv, "bf16"))
    done, elapsed, tokens = 0, 0.0, 0
    while elapsed < budget_s or done < 4:
        b = seqs[done % len(seqs)]
        i = int(rng.integers(case.H))
        t0 = time.perf_counter()
        omla.decode(C, R, case.seq_start, case.lens, args["q_nope"], args["q_rope"], args["w_uk"],
                    args["w_uv"], case.softmax_scale, case.rope_base, pairs=[(b, i)])
        elapsed += time.perf_counter() - t0
        tokens += int(case.lens[b])
        done += 1
        if done >= 4000:
            break
    # per (token, head) cost, scaled to the step's tokens x heads
    per_tok_head = elapsed / tokens
    step_s = per_tok_head * float(case.lens.sum()) * case.H
    return {"value": round(res["cache_bytes"] / step_s / 1e9, 6), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "step_seconds": round(step_s, 3),
            "sample": f"{done} (sequence, head) pairs of the workload ({tokens} token-heads, "
                      f"{elapsed:.1f} s of fp64 non-absorbed decode), scaled to {case.B} sequences x {case.H} heads"}


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
    par = sampled_parity(res)
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
        "kernel_ms": {k: round(v, 5) for k, v in res["prof"].items()},
        "ms_per_step_with_kernel_events": round(res["ms_step_profiled"], 5),
        "parity_sampled_max_err_over_rms": round(par, 6),
        "roofline": {"kernel": "splitk_decode (bf16 latent)", "bound": "hbm", "achieved": round(ach, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "per_launch_bytes": res["cache_bytes"], "avg_launch_ms": round(res["splitk_ms"], 5),
                     "stream_read_GBs": round(ceiling, 1), "frac_of_stream_read": round(ach / ceiling, 4)},
    }
    if a.extra:
        out["other_workloads"] = {}
        for name, ql in (("v3_b32_8k", 1), ("v3_b1_4k", 1), ("v3_b4_128k", 1), ("v3_b128_fp8", 1),
                         ("v3_b32_ragged", 4)):
            r = run_workload(m, torch, name, a.steps, a.warmup, q_len=ql)
            out["other_workloads"][name if ql == 1 else f"{name}_{ql}_query_tokens"] = workload_summary(r)
            del r
            torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(res, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
