#!/usr/bin/env python3
"""Benchmark of the attention forward on one MI355X.

One step is one pass of the whole hot path over one batch of seeded synthetic
input, with every input already resident in HBM:
  * decode leg -- FlashDecoding split-KV decode of a 128K-token cache (BNSD,
    B=1, 32 heads, D=128, bf16): stage 1 (fa_decode_splitkv) + the LSE
    combine (fa_combine), with the split plan fa_fwd would choose;
  * prefill leg -- mask-free prefill, BSND, B=2, 32 heads, S=4096, D=128, bf16
    (fa_fwd).
Each kernel launch is bracketed by HIP events on the stream it runs on, and the
median over the timed steps is reported (p10 / p90 beside it).  Before every
timed decode call a 1 GiB buffer is read outside the events, so the KV cache is
not served from the 256 MB of L2 + MALL.

The printed JSON line reports decode KV-read GB/s as ``value`` (and the prefill
TFLOP/s beside it), a ``roofline`` object for the dominant kernel (decode stage
1: K+V bytes per launch / its mean launch time, against 8 TB/s HBM) and one for
the prefill kernel (4*B*N*S^2*D flop per launch against 2.5 PFLOP/s bf16 MFMA),
and ``cpu_baseline``: the fp64 oracle timed on this host's cores on the same
decode workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
METRIC = "prefill attn TFLOP/s (%MFMA peak); decode KV GB/s (%HBM peak) on 1 MI355X"


# Headers every kernel source includes: a change to them changes the kernels too.
SHARED_HEADERS = ("fa_device.h", "fa_kernels.h", "fa_mfma.h")


# A string literal (kept), or a comment (dropped).
_C_TOKEN = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C/C++ source with its comments, trailing blanks and empty lines removed: an edit to
    comments alone leaves it unchanged."""
    src = _C_TOKEN.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    return "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())


def sha256_of(path):
    """Digest of the code (comments removed) of a kernel source together with the shared
    device headers beside it."""
    h = hashlib.sha256()
    for p in (path,) + tuple(os.path.join(os.path.dirname(path), n) for n in SHARED_HEADERS):
        with open(p, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
            h.update(b"\0")
    return h.hexdigest()


def stored_traffic(kernel_src: str, name: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on this source
    (the kernel file and the shared headers)."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and not line.startswith("#"):
            vals[parts[0]] = parts[1]
    if vals.get("source_sha256") != sha256_of(kernel_src):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--legs", default="decode,prefill", help="comma list of decode,prefill")
    ap.add_argument("--chunk", type=int, default=0, help="decode chunk (tokens); 0 = planner")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run a plain 1 GiB device copy per step (counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-workload report of the other configurations")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the attention path runs on one GPU; --gpus must be 1 (sharding across GPUs is not implemented)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import fa_synth
    import split_kv_decode_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    fa.load()
    legs = [x for x in args.legs.split(",") if x]
    stream = torch.cuda.current_stream()

    def dev16(bits, dtype):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)

    t_gen = time.time()
    dec = pre = None
    if "decode" in legs:
        dinp = fa_synth.make(fa_synth.WORKLOADS["decode_128k"])
        ds = dinp.spec
        dq, dk, dv = (dev16(x, ds.dtype) for x in (dinp.q, dinp.k, dinp.v))
        dp = fa.params_for(dq, dk, layout=ds.layout, scale=ds.softmax_scale)
        splits, chunk, ws_bytes = fa.fa_splitkv_plan(dp, 0, args.chunk)
        rows = ds.B * ds.QN
        o_part = torch.empty((rows * splits * ds.D,), dtype=torch.float32, device=dev)
        m_part = torch.empty((rows * splits,), dtype=torch.float32, device=dev)
        l_part = torch.empty((rows * splits,), dtype=torch.float32, device=dev)
        dout = torch.empty_like(dq)
        dlse = torch.empty((rows,), dtype=torch.float32, device=dev)
        kv_bytes = 2 * ds.B * ds.KVN * ds.KVS * ds.D * 2      # K and V, bf16, every row valid
        qo_bytes = 2 * rows * ds.D * 2                         # q in, out back
        dec = dict(inp=dinp, q=dq, k=dk, v=dv, p=dp, splits=splits, chunk=chunk,
                   o=o_part, m=m_part, l=l_part, out=dout, lse=dlse,
                   kv_bytes=kv_bytes, qo_bytes=qo_bytes)
        del dinp
    if "prefill" in legs:
        pinp = fa_synth.make(fa_synth.WORKLOADS["prefill_4k"])
        ps = pinp.spec
        pq, pk, pv = (dev16(x, ps.dtype) for x in (pinp.q, pinp.k, pinp.v))
        pp = fa.params_for(pq, pk, layout=ps.layout, scale=ps.softmax_scale)
        pout = torch.empty_like(pq)
        plse = torch.empty((ps.B, ps.QN, ps.QS), dtype=torch.float32, device=dev)
        flops = 4.0 * ps.B * ps.QN * ps.QS * ps.KVS * ps.D
        pre = dict(spec=ps, q=pq, k=pk, v=pv, p=pp, out=pout, lse=plse, flops=flops)
        del pinp
    # Read before every timed decode call, outside its events, so the 256 MB of
    # L2 + MALL holds none of the KV cache when the call starts.  A read leaves
    # the caches clean; a write would leave dirty lines whose write-back then
    # competes with the decode's reads.
    flush = torch.ones((1 << 28,), dtype=torch.float32, device=dev) if dec is not None else None
    copy_src = copy_dst = None
    if args.copy_calibrate:
        copy_src = torch.ones((1 << 29,), dtype=torch.int16, device=dev)  # 1 GiB
        copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    def step(ev):
        if dec is not None:
            flush.sum()
            ev[0].record(stream)
            fa.fa_decode_splitkv(dec["p"], dec["splits"], dec["chunk"], dec["q"], dec["k"], dec["v"],
                                 dec["o"], dec["m"], dec["l"], stream)
            ev[1].record(stream)
            fa.fa_combine(dec["p"], dec["splits"], dec["o"], dec["m"], dec["l"], dec["out"],
                          dec["lse"], stream)
            ev[2].record(stream)
        if pre is not None:
            ev[3].record(stream)
            fa.fa_fwd(pre["p"], pre["q"], pre["k"], pre["v"], pre["out"], pre["lse"], None, 0, stream)
            ev[4].record(stream)
        if copy_src is not None:
            copy_dst.copy_(copy_src)

    def new_events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    for _ in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()

    events = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    def stats_ms(a, b):
        t = np.array([ev[a].elapsed_time(ev[b]) for ev in events])
        return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))

    def median_ms(a, b):  # p10 / p90 are reported beside it
        return stats_ms(a, b)[0]

    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) bf16, RNE-rounded)"}
    config = {"workload": "+".join({"decode": "decode_128k", "prefill": "prefill_4k"}[x] for x in legs),
              "parallelism": "single GPU"}
    csrc = os.path.join(ROOT, "split_kv_decode_amd", "csrc")
    if dec is not None:
        s1 = median_ms(0, 1)
        cb = median_ms(1, 2)
        leg = s1 + cb
        value = (dec["kv_bytes"] + dec["qo_bytes"]) / (leg * 1e-3) / 1e9
        s1_gbs = (dec["kv_bytes"] + dec["qo_bytes"]) / (s1 * 1e-3) / 1e9
        traffic = stored_traffic(os.path.join(csrc, "fa_decode.hip"), "decode_stage1_128k")
        out["value"] = round(value, 2)
        legs_t = np.array([ev[0].elapsed_time(ev[2]) for ev in events])
        out["decode"] = {"workload": "decode_128k: BNSD B=1 Q_N=KV_N=32 Q_S=1 KV_S=131072 D=128 bf16",
                         "num_splits": dec["splits"], "chunk": dec["chunk"],
                         "stage1_ms": round(s1, 5), "combine_ms": round(cb, 5),
                         "leg_ms": round(leg, 5), "kv_gbs": round(value, 2),
                         "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                         "leg_ms_p10_p90": [round(float(np.percentile(legs_t, 10)), 5),
                                            round(float(np.percentile(legs_t, 90)), 5)],
                         "timing": "median over the timed steps; a 1 GiB buffer is read before each "
                                   "decode call, outside its events, so no KV is cached"}
        out["roofline"] = {"kernel": "decode_stage1_kernel<BF16,128,1,0,false,false>", "bound": "hbm",
                           "achieved": round(s1_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(s1_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                           "algorithmic_bytes_per_launch": dec["kv_bytes"] + dec["qo_bytes"]}
        config.update({"decode_B": 1, "decode_heads": 32, "decode_kv_seq": 131072, "head_dim": 128})
    if pre is not None:
        pm = median_ms(3, 4)
        tflops = pre["flops"] / (pm * 1e-3) / 1e12
        ps = pre["spec"]
        traffic = stored_traffic(os.path.join(csrc, "fa_prefill.hip"), "prefill_4k")
        _, p10, p90 = stats_ms(3, 4)
        out["prefill"] = {"workload": "prefill_4k: BSND B=2 N=32 S=4096 D=128 bf16, no mask",
                          "ms": round(pm, 5), "ms_p10_p90": [round(p10, 5), round(p90, 5)],
                          "tflops": round(tflops, 2),
                          "frac_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
        out["roofline_prefill"] = {"kernel": "prefill_il_kernel<BF16,128,0,true,false> (persistent)", "bound": "mfma",
                                   "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                                   "traffic": traffic, "algorithmic_flop_per_launch": pre["flops"]}
        if dec is None:
            out["value"] = round(tflops, 2)
            out["unit"] = "TFLOP/s"
        config.update({"prefill_B": ps.B, "prefill_heads": ps.QN, "prefill_seq": ps.QS})
    out["config"] = config
    if pre is not None:
        run = lambda: fa.fa_fwd(pre["p"], pre["q"], pre["k"], pre["v"], pre["out"], pre["lse"], None, 0, stream)
        out["shader_clock"] = clock_under_load(run, torch, "the prefill_4k kernel")
    elif dec is not None:
        run = lambda: fa.fa_decode_splitkv(dec["p"], dec["splits"], dec["chunk"], dec["q"], dec["k"], dec["v"],
                                           dec["o"], dec["m"], dec["l"], stream)
        out["shader_clock"] = clock_under_load(run, torch, "the decode_128k stage 1")

    if dec is not None and not args.no_cpu_baseline:
        import oracle
        inp = dec["inp"]
        prob = oracle.Problem.from_inputs(inp)
        threads = oracle.default_threads()
        n, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds:
            t1 = time.perf_counter()
            oracle.attention_rows(prob, inp.q, inp.k, inp.v, None, threads)
            t_cpu += time.perf_counter() - t1
            n += 1
        cpu_gbs = n * (dec["kv_bytes"] + dec["qo_bytes"]) / t_cpu / 1e9
        out["cpu_baseline"] = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": threads,
                               "nproc": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
                               "kind": "oracle",
                               "sample": f"the whole decode_128k workload (32 rows x 131072 keys), "
                                         f"{n} pass(es) in {t_cpu:.1f} s, fp64"}
    if not args.no_extra:
        out["workloads"] = extra_workloads(fa, fa_synth, np, torch, dev16, stream)
    out["setup_s"] = round(t_gen, 1)
    print(json.dumps(out))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_sclk_mhz():
    """Current shader clock from the driver's sysfs DPM table (the line marked '*'), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def clock_under_load(fn, torch, what, seconds=0.5):
    """Shader clock while fn() keeps the GPU busy, read after the timed steps (outside them):
    batches of launches are queued and the driver's current DPM clock is sampled between them."""
    if read_sclk_mhz() is None:
        return {"available": False, "why": "no readable pp_dpm_sclk in /sys/class/drm on this host"}
    samples = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(16):
            fn()
        time.sleep(0.002)
        mhz = read_sclk_mhz()
        if mhz is not None:
            samples.append(mhz)
        torch.cuda.synchronize()
    samples.sort()
    return {"available": True, "mhz_median": samples[len(samples) // 2], "mhz_min": samples[0],
            "mhz_max": samples[-1], "samples": len(samples),
            "source": f"sysfs pp_dpm_sclk, sampled while {what} ran in an untimed loop after the timed steps"}


def timed(fn, torch, np, stream, warmup, iters, flush=None, warm_s=0.25):
    """Median ms of fn() over iters calls, each between events on the stream; with a flush
    buffer, the buffer is read before each call, outside its events.  The warmup runs at
    least `warmup` calls and at least warm_s seconds: the GPU idles while the next
    workload's inputs are generated on the host, and its clock needs some tens of
    milliseconds of load to come back up."""
    t_end = time.perf_counter() + warm_s
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for a, b in evs:
        if flush is not None:
            flush.sum()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def extra_workloads(fa, fa_synth, np, torch, dev16, stream, warmup=3, iters=20):
    """Time the other configurations with fa_fwd (events on the launch stream; decode calls
    start with no KV in L2 or MALL)."""
    res = {}
    flush = torch.ones((1 << 28,), dtype=torch.float32, device=torch.device("cuda:0"))
    # (workload, mask mode override, paged cache (kv_layout, block_size) or None)
    cases = [("prefill_small", None, None), ("decode_gqa", None, None),
             ("decode_gqa", None, ("PA_BBND", 128)), ("decode_128k", None, ("PA_BNBD", 128)),
             ("prefill_causal", "bool", None), ("prefill_causal", "causal", None),
             ("prefill_4k", "window", None), ("prefill_gqa_long", None, None),
             ("prefill_4k_d256", None, None), ("prefill_4k_d256", "window", None)]
    window = (1024, 0)  # sliding window of the last 1025 keys
    for name, mode, paging in cases:
        inp = fa_synth.make(fa_synth.WORKLOADS[name])
        s = inp.spec
        block_table = None
        if paging is None:
            q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
        else:
            if inp.lens is None:  # a paged cache always carries per-batch lengths
                inp.lens = np.full(s.B, s.KVS, dtype=np.int64)
            kp, vp, table, nblocks = fa_synth.to_paged(inp, paging[1], paging[0])
            q, k, v = dev16(inp.q, s.dtype), dev16(kp, s.dtype), dev16(vp, s.dtype)
            block_table = torch.from_numpy(table).to(q.device)
            del kp, vp
        lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(q.device)
        m = mode or {"none": "none", "causal": "causal", "bool_causal": "bool"}[s.mask]
        mask = torch.from_numpy(inp.mask).to(q.device) if m == "bool" else None
        if paging is None:
            p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens,
                              mask=mask, mask_stride=inp.mask_strides, causal=(m == "causal"),
                              window=window if m == "window" else None)
        else:
            p = fa.make_params(s.B, s.QN, 1, s.KVS, s.D, num_kv_heads=s.KVN, layout=s.layout,
                               dtype=s.dtype, scale=s.softmax_scale, actual_seq_lengths=lens,
                               kv_layout=paging[0], block_table=block_table, block_size=paging[1],
                               max_blocks_per_seq=block_table.shape[1], num_blocks=nblocks)
        out = torch.empty_like(q)
        lse = torch.empty((s.B, s.QN, s.QS), dtype=torch.float32, device=q.device)
        nbytes = fa.fa_workspace_size(p)
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
        ms = timed(lambda: fa.fa_fwd(p, q, k, v, out, lse, ws, nbytes, stream), torch, np, stream,
                   warmup, iters, flush if s.QS == 1 else None)
        key = name if mode is None else f"{name}_{mode}"
        if mode == "window":
            key = f"{name}_window{window[0]}_{window[1]}"
        if paging is not None:
            key = f"{name}_paged_{paging[0]}_bs{paging[1]}"
        if s.QS == 1:
            L = np.full(s.B, s.KVS) if inp.lens is None else np.clip(inp.lens, 0, s.KVS)
            nb = float(L.sum()) * s.KVN * s.D * 2 * 2 + 2 * s.B * s.QN * s.D * 2
            gbs = nb / (ms * 1e-3) / 1e9
            res[key] = {"ms": round(ms, 5), "kv_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes": nb, "doc": s.doc,
                        "kv_cache": "contiguous" if paging is None else f"{paging[0]}, block_size {paging[1]}"}
        else:
            S = s.QS
            if m == "none" and inp.lens is None:
                fl = 4.0 * s.B * s.QN * S * s.KVS * s.D
            elif m == "window":  # row i sees keys max(0, i - wl) .. min(L - 1, i + wr)
                L = np.full(s.B, s.KVS) if inp.lens is None else np.clip(inp.lens, 0, s.KVS)
                i = np.arange(S, dtype=np.float64)
                pairs = sum(np.clip(np.minimum(Lb - 1, i + window[1]) - np.maximum(0, i - window[0]) + 1,
                                    0, None).sum() for Lb in L)
                fl = 4.0 * s.QN * s.D * float(pairs)
            else:
                L = np.full(s.B, s.KVS) if inp.lens is None else np.clip(inp.lens, 0, s.KVS).astype(np.float64)
                if m == "none":
                    pairs = L * S
                else:  # causal: row i sees min(i + 1, L) keys
                    pairs = L * (L + 1) / 2 + np.maximum(S - L, 0) * L
                fl = 4.0 * s.QN * s.D * float(np.sum(pairs))
            tf = fl / (ms * 1e-3) / 1e12
            res[key] = {"ms": round(ms, 5), "tflops": round(tf, 2),
                        "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flop": fl, "doc": s.doc}
            if mode is not None:  # the spec's own mask is replaced by the mode timed here
                res[key]["mask_timed"] = {"bool": "boolean mask tensor (upper-triangular)",
                                          "causal": "causal flag, no mask tensor",
                                          "window": f"sliding window ({window[0]}, {window[1]})"}[mode]
        del q, k, v, out, lse, ws, mask, inp, block_table
        torch.cuda.empty_cache()
    res.update(packed_workload(fa, fa_synth, np, torch, dev16, stream, warmup, iters))
    res.update(fused_decode(fa, fa_synth, np, torch, dev16, stream, warmup, iters, flush))
    res.update(split_decode_workloads(fa, fa_synth, np, torch, dev16, stream, warmup, iters, flush))
    return res


def split_decode_workloads(fa, fa_synth, np, torch, dev16, stream, warmup, iters, flush):
    """Query work too small to occupy the chip, which fa_fwd runs as split-KV on the general
    matrix-core stage 1 (rows = query head x position) plus the combine: one query position
    under a boolean mask, and eight positions against a 64K cache, without a mask and with a
    causal band aligned to the cache's end given as a boolean tensor (the top-left causal
    flag would leave those rows eight keys)."""
    res = {}
    rng = np.random.default_rng(1012)
    S128, S64 = 131072, 65536
    pad = (rng.random(S128) < 0.125) | (np.arange(S128) >= S128 - 4096)  # dropped keys + a padded tail
    band = np.arange(S64)[None, :] > (S64 - 8 + np.arange(8))[:, None]   # key j hidden from row i
    cases = [
        (fa_synth.Spec("decode_128k_bool_mask", "BNSD", B=1, QN=32, KVN=32, QS=1, KVS=S128, D=128,
                       dtype="bf16", seed=1003,
                       doc="decode_128k (BNSD, B=1, N=32, KV_S=131072, D=128, bf16 N(0,1)) with a "
                           "(B,1,1,S) boolean mask: 1/8 of the keys dropped at random and the last "
                           "4096 hidden"),
         pad.astype(np.uint8).reshape(1, S128), (S128, 0, 0, 1)),
        (fa_synth.Spec("decode_q8_65k", "BSND", B=1, QN=32, KVN=8, QS=8, KVS=S64, D=128, dtype="bf16",
                       seed=1013, doc="eight query positions, BSND, B=1, Q_N=32, KV_N=8, KV_S=65536, "
                                      "D=128, bf16 N(0,1), no mask"),
         None, (0, 0, 0, 0)),
        (fa_synth.Spec("decode_q8_65k_tail_causal", "BSND", B=1, QN=32, KVN=8, QS=8, KVS=S64, D=128,
                       dtype="bf16", seed=1013,
                       doc="eight query positions against KV_S=65536 (BSND, B=1, Q_N=32, KV_N=8, "
                           "D=128, bf16 N(0,1)) with a (1,1,8,S) boolean mask: row i sees keys "
                           "j <= S - 8 + i"),
         band.astype(np.uint8), (8 * S64, 0, S64, 1)),
    ]
    for spec, mask_np, strides in cases:
        inp = fa_synth.make(spec)
        q, k, v = (dev16(x, spec.dtype) for x in (inp.q, inp.k, inp.v))
        mask = None if mask_np is None else torch.from_numpy(np.ascontiguousarray(mask_np)).to(q.device)
        p = fa.params_for(q, k, layout=spec.layout, scale=spec.softmax_scale, mask=mask,
                          mask_stride=strides)
        out = torch.empty_like(q)
        lse = torch.empty((spec.B, spec.QN, spec.QS), dtype=torch.float32, device=q.device)
        nbytes = fa.fa_workspace_size(p)
        ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
        ms = timed(lambda: fa.fa_fwd(p, q, k, v, out, lse, ws, nbytes, stream), torch, np, stream,
                   warmup, iters, flush)
        nb = (2.0 * spec.B * spec.KVN * spec.KVS * spec.D * 2 + 2 * spec.B * spec.QN * spec.QS * spec.D * 2
              + (0 if mask_np is None else mask_np.size))
        gbs = nb / (ms * 1e-3) / 1e9
        res[spec.name] = {"ms": round(ms, 5), "kv_gbs": round(gbs, 1),
                          "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": nb,
                          "path": fa.fa_describe(p).split(" -> ")[1], "doc": spec.doc}
        del q, k, v, out, lse, ws, mask, inp
        torch.cuda.empty_cache()
    return res


def fused_decode(fa, fa_synth, np, torch, dev16, stream, warmup, iters, flush):
    """The single-launch split-KV (fa_decode_fused) on the two decode workloads, with the
    fused plan (fa_decode_fused_plan), for comparison with fa_fwd's stage 1 + combine."""
    res = {}
    for name in ("decode_128k", "decode_gqa"):
        inp = fa_synth.make(fa_synth.WORKLOADS[name])
        s = inp.spec
        q, k, v = (dev16(x, s.dtype) for x in (inp.q, inp.k, inp.v))
        lens = None if inp.lens is None else torch.from_numpy(inp.lens).to(q.device)
        p = fa.params_for(q, k, layout=s.layout, scale=s.softmax_scale, actual_seq_lengths=lens)
        sp, ch, nbytes = fa.fa_decode_fused_plan(p)
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device=q.device)
        out = torch.empty_like(q)
        lse = torch.empty((s.B, s.QN, 1), dtype=torch.float32, device=q.device)
        ms = timed(lambda: fa.fa_decode_fused(p, sp, ch, q, k, v, ws, nbytes, out, lse, stream), torch,
                   np, stream, warmup, iters, flush)
        L = np.full(s.B, s.KVS) if inp.lens is None else np.clip(inp.lens, 0, s.KVS)
        nb = float(L.sum()) * s.KVN * s.D * 2 * 2 + 2 * s.B * s.QN * s.D * 2
        gbs = nb / (ms * 1e-3) / 1e9
        res[f"{name}_fused_single_launch"] = {
            "ms": round(ms, 5), "kv_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": nb, "num_splits": sp, "doc": s.doc + "; fa_decode_fused (one launch)"}
        del q, k, v, ws, out, lse, inp
        torch.cuda.empty_cache()
    return res


def packed_workload(fa, fa_synth, np, torch, dev16, stream, warmup, iters):
    """The ragged causal prefill in the packed (TND) layout, schedule kernel included."""
    x = fa_synth.make_packed(**fa_synth.PACKED_WORKLOADS["prefill_varlen"])
    q, k, v = dev16(x.q, x.dtype), dev16(x.k, x.dtype), dev16(x.v, x.dtype)
    cu_q = torch.from_numpy(x.cu_q).to(q.device)
    cu_kv = torch.from_numpy(x.cu_kv).to(q.device)
    p = fa.params_for(q, k, layout="TND", scale=x.scale, causal=True, cu_seqlens_q=cu_q,
                      cu_seqlens_kv=cu_kv)
    out = torch.empty_like(q)
    lse = torch.empty((p.q_seq, p.num_heads), dtype=torch.float32, device=q.device)
    nbytes = fa.fa_workspace_size(p)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    ms = timed(lambda: fa.fa_fwd(p, q, k, v, out, lse, ws, nbytes, stream), torch, np, stream,
               warmup, iters)
    L = x.q_lens.astype(np.float64)
    fl = 4.0 * x.QN * x.D * float(np.sum(L * (L + 1) / 2))
    tf = fl / (ms * 1e-3) / 1e12
    return {"prefill_varlen_causal": {
        "ms": round(ms, 5), "tflops": round(tf, 2), "frac_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "flop": fl, "doc": "packed (TND) causal prefill, 16 sequences of U{256..8192} tokens "
                           f"(total {int(x.cu_q[-1])}), Q_N=32, KV_N=8, D=128, bf16; "
                           "includes the work-list kernel"}}


if __name__ == "__main__":
    main()
