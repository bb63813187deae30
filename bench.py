"""Throughput of the packed-bitmask apply on one MI355X.

One step = one in-place apply of a packed int32 allow-mask to bf16 logits
[256, 128256] with vocab_size 128000 and 128 random unique row indices
(batch 256 x 128k vocab is the shape the logits-processor page benchmarks;
the vocab/padding and index rules are XGrammar "Bitmask Operations").

Metric: effective HBM bandwidth = algorithmic bytes per step / time per step,
algorithmic bytes = mask words of the processed rows (R * ceil(V/32) * 4)
+ one write pass over their logits (R * V * 2).

Timing: inputs sit in HBM; the timed region rotates over enough independent
buffer sets (> 2 x the 256 MB Infinity Cache) that no step finds its data in
a cache.  The K launches are captured once in a HIP graph and replayed, so
the host's launch rate does not pace the GPU; HIP events on the launch
stream bracket the replay.  The CPU baseline is the oracle's plain C loop
on one host core over repeated passes of the same workload.

Besides the headline, the one JSON line carries: the same steps' rate in
HBM traffic (from the committed counter summary), a warm figure (one buffer
set, cache-resident, not HBM), each kernel variant cold, fill and copy
ceilings (two of them moving the apply's physical bytes: a torch copy and
this library's out-of-place apply with an all-allowed mask), the gated apply
with its report, one GPU's share under a vocabulary split, the host-memory
path, mask upload behind a forward pass, the fused sampler against a
stock-torch sampler and at small batches, and the oracle on all host cores
and in pure Python.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--variant auto]
       python bench.py --all-configs       (every workload, next to a plain fill)
       python bench.py --copy-calibration  (plain copies, for scaling HBM counters)
       python bench.py --sampler-calls N   (N eager sampler calls per mode, for counters)
       python bench.py --split-calls N     (N eager small-batch filtered sampler calls, for kernel traces)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "effective HBM GB/s (% of MI355X peak) for bitmask apply, B=256 V=128000 bf16"
PEAK_GBPS = 8000.0          # MI355X HBM3E, published
INFINITY_CACHE = 256 << 20  # bytes


def cold_sets(touched: int, cap: int = 0) -> int:
    """Buffer sets a cold rotation needs: more than twice the Infinity Cache
    in the bytes that one launch touches (not the bytes each set holds: a
    launch that reads half of a set's rows leaves the other half out of the
    cache's traffic).  cap > 0 bounds the count for tiny launches, which then
    stay cache-resident."""
    n = max(2, math.ceil(2 * INFINITY_CACHE / max(1, touched)))
    return min(cap, n) if cap else n


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--variant", default="auto", choices=["auto", "scalar", "vec", "wronly", "vec_resident"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU work for the oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the warm, per-variant and ceiling figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain 64 MiB device copies (for scaling FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline line, print one line timing the apply on each of the five "
                         "workloads (cold) next to a plain fill of the same bytes")
    ap.add_argument("--sampler-calls", type=int, default=0, metavar="N",
                    help="only call the fused sampler N times per mode on its two shapes, eagerly (for hardware "
                         "counters)")
    ap.add_argument("--split-calls", type=int, default=0, metavar="N",
                    help="only call the fused sampler N times per case on the first 1 and 16 rows of the B=256 "
                         "bf16 shape with top-k 50 and top-p 0.9, eagerly, with the workspace that splits filtered "
                         "rows (for kernel traces)")
    return ap.parse_args()


# the sources that define the apply kernels, their shapes and launches
KERNEL_SOURCES = [ROOT / "packed_logit_bitmask_amd" / "csrc" / "apply_kernels.h",
                  ROOT / "packed_logit_bitmask_amd" / "csrc" / "host_checks.h",
                  ROOT / "packed_logit_bitmask_amd" / "csrc" / "mi_bitmask.hip"]
PMC_SUMMARY = ROOT / "profiles" / "inplace_vec_mixed_bf16_pmc.md"


def counted_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary.

    None when the summary is missing or was taken on kernel sources other
    than the ones in this tree.
    """
    import hashlib
    import re

    if not PMC_SUMMARY.exists():
        return None
    text = PMC_SUMMARY.read_text()
    m_bytes = re.search(r"^traffic_bytes_per_dispatch:\s*(\d+)", text, re.M)
    m_sha = re.search(r"^kernel_source_sha256_16:\s*([0-9a-f]+)", text, re.M)
    if not (m_bytes and m_sha):
        return None
    h = hashlib.sha256(b"".join(p.read_bytes() for p in KERNEL_SOURCES)).hexdigest()[:16]
    return int(m_bytes.group(1)) if h == m_sha.group(1) else None


def copy_calibration():
    """Five plain copies of 64 MiB, caches flushed between them by a 600 MiB fill.

    Under rocprofv3 --pmc the copy kernel's FETCH_SIZE and WRITE_SIZE per
    dispatch, against the 65536 KiB it really reads and writes, give the
    factors that turn the counters into bytes.
    """
    import torch

    n = 64 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    flush = torch.empty(600 << 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    for k in range(5):
        flush.fill_(k)
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "dispatches": 5}}), flush=True)


def sampler_calls(n):
    """N eager calls of the fused sampler per mode on the three shapes the sampler figures use.

    Under rocprofv3 --pmc each call is one dispatch, in the order printed, or
    two where a large batch hands out its dense rows first (row_classes, then
    the draw).
    """
    import numpy as np
    import torch

    import packed_logit_bitmask_amd as mb
    import workloads

    dev = torch.device("cuda:0")
    for label, wl, fp32 in (("B256_V128000_bf16", workloads.mixed_bf16(n_indices=0), False),
                            ("B1024_V32000_fp16", workloads.verify_fp16(), False),
                            ("B256_V128000_fp32", workloads.mixed_bf16(n_indices=0), True)):
        tdt = torch.bfloat16 if wl.dtype == "bfloat16" else torch.float16
        x = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(tdt)
        if fp32:
            x = x.float().contiguous()
        m = torch.from_numpy(wl.mask).to(dev)
        tok = torch.empty(wl.rows, dtype=torch.int64, device=dev)
        for mode, kw in SAMPLER_MODES:
            for k in range(n):
                mb.mi_apply_bitmask_sample(x, m, wl.vocab_size, seed=1, offset=k, out=tok, **kw)
            torch.cuda.synchronize()
            print(json.dumps({"sampler_calls": {"shape": label, "mode": mode, "calls": n}}), flush=True)


def split_calls(n):
    """N eager calls of the fused sampler with its split-row workspace, per case.

    Cases: the first B = 1 and 16 rows of the B=256 bf16 sampler shape, top-k
    50 and top-p 0.9, in that order.  Each call is five dispatches: the
    workspace clear, split_hist, split_search, the segmented draw
    (sample_rows) and the token conversion.
    """
    import numpy as np
    import torch

    import packed_logit_bitmask_amd as mb
    import workloads

    dev = torch.device("cuda:0")
    wl = workloads.mixed_bf16(n_indices=0)
    x = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    m = torch.from_numpy(wl.mask).to(dev)
    for B in (1, 16):
        tok = torch.empty(B, dtype=torch.int64, device=dev)
        ws = torch.empty(mb.sample_workspace_bytes(torch.bfloat16, B, wl.vocab_size), dtype=torch.uint8, device=dev)
        for mode, kw in (("top_k_50", dict(top_k=50)), ("top_p_0.9", dict(top_p=0.9))):
            for k in range(n):
                mb.mi_apply_bitmask_sample(x[:B], m[:B], wl.vocab_size, seed=1, offset=k, out=tok, workspace=ws, **kw)
            torch.cuda.synchronize()
            print(json.dumps({"split_calls": {"rows": B, "mode": mode, "calls": n}}), flush=True)


def all_configs():
    """The apply on each of the five workloads, cold, next to a plain fill.

    Per workload: K buffer sets with K x (logits + mask [+ out]) above
    2 x the Infinity Cache (one set when a single set is larger; at most 64,
    so the two launch-bound workloads of well under 1 MB stay in the
    caches), a graph of
    launches cycling through them, HIP events around its second replay on
    the launch stream.  The fill ceiling is torch's fill of a buffer of the
    workload's effective bytes under the same rotation; the copy ceiling a
    torch copy that moves the same total bytes, half read and half written.
    Parity for every workload is in the GPU tests, not here.
    """
    import numpy as np
    import torch

    import packed_logit_bitmask_amd as mb
    import workloads

    mb.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    tdt = {"float32": (np.int32, torch.float32), "float16": (np.int16, torch.float16),
           "bfloat16": (np.int16, torch.bfloat16)}
    out = []
    for make in (workloads.tiny, workloads.tail_bf16, workloads.mixed_bf16, workloads.verify_fp16,
                 workloads.large_fp32):
        wl = make()
        ndt, dt = tdt[wl.dtype]
        esize = wl.logits.dtype.itemsize
        rows, cols = wl.logits.shape
        V = wl.vocab_size if wl.vocab_size is not None else min(cols, 32 * wl.mask.shape[1])
        R = len(wl.indices) if wl.indices is not None else rows
        eff = effective_bytes(R, V, esize, wl.op == "out")
        # one launch touches its effective bytes: the processed rows' logits
        # (and output) and mask words
        nsets = 1 if eff > 2 * INFINITY_CACHE else cold_sets(eff, cap=64)
        host = torch.from_numpy(wl.logits.view(ndt))
        sets = []
        for _ in range(nsets):
            x = host.to(dev).view(dt)
            m = torch.from_numpy(wl.mask).to(dev)
            i = torch.from_numpy(wl.indices).to(dev) if wl.indices is not None else None
            o = torch.empty_like(x) if wl.op == "out" else None
            sets.append((x, m, i, o))
        steps = 1000 if eff < 1e6 else max(50, min(400, int(4e9 / eff)))
        if wl.op == "out":
            fn = lambda k: mb.mi_apply_bitmask_out(sets[k % nsets][0], sets[k % nsets][1], sets[k % nsets][3],
                                                   wl.vocab_size, sets[k % nsets][2], wl.fill_value)
        else:
            fn = lambda k: mb.mi_apply_bitmask_inplace(sets[k % nsets][0], sets[k % nsets][1], wl.vocab_size,
                                                       sets[k % nsets][2], wl.fill_value)
        ms = graph_ms(torch, fn, steps, stream)
        del sets
        torch.cuda.empty_cache()
        fsets = min(64, max(1, math.ceil(2 * INFINITY_CACHE / eff)))
        bufs = [torch.empty(eff, dtype=torch.uint8, device=dev) for _ in range(fsets)]
        fill_ms = graph_ms(torch, lambda k: bufs[k % fsets].fill_(7), steps, stream)
        del bufs
        torch.cuda.empty_cache()
        # a plain copy that reads half the effective bytes and writes them:
        # the same total traffic, half of it reads
        half = max(1, eff // 2)
        csets = min(64, max(1, math.ceil(2 * INFINITY_CACHE / eff)))
        cbufs = [(torch.empty(half, dtype=torch.uint8, device=dev).fill_(1),
                  torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(csets)]
        copy_ms = graph_ms(torch, lambda k: cbufs[k % csets][1].copy_(cbufs[k % csets][0]), steps, stream)
        del cbufs
        torch.cuda.empty_cache()
        gbps = eff / (ms * 1e-3) / 1e9
        fill_gbps = eff / (fill_ms * 1e-3) / 1e9
        copy_gbps = 2 * half / (copy_ms * 1e-3) / 1e9
        out.append({"workload": wl.name, "op": wl.op, "dtype": wl.dtype, "shape": [rows, cols], "vocab_size": V,
                    "rows_processed": R, "effective_bytes": eff, "buffer_sets": nsets, "launches": steps,
                    "us_per_launch": round(ms * 1e3, 3), "GBps": round(gbps, 1),
                    "frac_of_peak": round(gbps / PEAK_GBPS, 4), "fill_ceiling_GBps": round(fill_gbps, 1),
                    "frac_of_fill_ceiling": round(gbps / fill_gbps, 4), "copy_ceiling_GBps": round(copy_gbps, 1),
                    "frac_of_copy_ceiling": round(gbps / copy_gbps, 4), "variant": "auto"})
        print(f"# {wl.name}: {ms * 1e3:.3f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
    print(json.dumps({"mode": "all_configs", "peak_GBps": PEAK_GBPS, "configs": out}), flush=True)


def effective_bytes(rows: int, vocab: int, esize: int, out_of_place: bool = False) -> int:
    words = (vocab + 31) // 32
    return rows * words * 4 + rows * vocab * esize * (2 if out_of_place else 1)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.all_configs:
        all_configs()
        return
    if args.sampler_calls > 0:
        sampler_calls(args.sampler_calls)
        return
    if args.split_calls > 0:
        split_calls(args.split_calls)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU (--gpus 1): the apply has no cross-GPU step, and each GPU of a "
              "larger job would run the same calls on its own rows.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import packed_logit_bitmask_amd as mb
    import workloads

    mb.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = workloads.mixed_bf16()
    R, V = len(wl.indices), wl.vocab_size
    eff = effective_bytes(R, V, 2)
    set_bytes = wl.logits.nbytes + wl.mask.nbytes
    nsets = cold_sets(eff)  # a launch touches only the indexed rows: eff bytes

    host_logits = torch.from_numpy(wl.logits.view(np.int16))
    sets = []
    for _ in range(nsets):
        x = host_logits.to(dev).view(torch.bfloat16)
        m = torch.from_numpy(wl.mask).to(dev)
        i = torch.from_numpy(wl.indices).to(dev)
        sets.append((x, m, i))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def timed(variant, steps, warmup, rotate=True):
        use = sets if rotate else sets[:1]

        def one(k):
            x, m, i = use[k % len(use)]
            mb.mi_apply_bitmask_inplace(x, m, V, i, -math.inf, variant=variant)

        with torch.cuda.stream(stream):
            for k in range(warmup):
                one(k)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for k in range(steps):
                one(k)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()  # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        del g
        return ms / steps

    ms_step = timed(args.variant, args.steps, args.warmup, rotate=True)
    gbps = eff / (ms_step * 1e-3) / 1e9
    print(f"# headline: {ms_step * 1e3:.3f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)

    extras = {}

    def phase(name, value):
        extras[name] = value
        print(f"# {name} done", file=sys.stderr, flush=True)

    if not args.no_extras:
        warm = timed(args.variant, args.steps, 10, rotate=False)
        warm_res = timed("vec_resident", args.steps, 10, rotate=False)
        extras["warm_cache_resident"] = {
            "note": "one buffer set reused every step: logits and mask stay in the 256 MB Infinity Cache; "
                    "not an HBM figure",
            "ms_per_step": warm, "GBps": eff / (warm * 1e-3) / 1e9,
            "vec_resident": {"ms_per_step": warm_res, "GBps": eff / (warm_res * 1e-3) / 1e9}}
        per = {}
        for var in ("scalar", "vec", "wronly", "vec_resident"):
            t = timed(var, args.steps, 10, rotate=True)
            per[var] = {"ms_per_step": t, "GBps": eff / (t * 1e-3) / 1e9}
        phase("variants_cold", per)
        phase("ceiling_cold", ceilings(torch, dev, eff, nsets, args.steps, stream, rmw_bytes=R * V * 2))
        extras["ceiling_cold"]["own_copy_same_rows"] = own_copy(torch, dev, mb, R, wl.logits.shape[1],
                                                                 wl.mask.shape[1], args.steps, stream)
        phase("gated_rows_cold", gated_rows(torch, dev, mb, workloads, args.steps, stream))
        phase("out_of_place_index_list_cold", out_of_place_listed(torch, dev, mb, workloads, args.steps, stream))
        phase("vocab_shard_tp8_cold", vocab_shard(torch, dev, mb, wl, args.steps, stream))
        phase("host_path", host_path(torch, mb, wl, eff))
        phase("mask_upload_overlap", upload_overlap(torch, dev, mb, wl))
        phase("fused_sampler_cold", sampler_times(torch, dev, mb, workloads, stream))
        phase("fused_sampler_small_batch_cache_resident", sampler_small_batch(torch, dev, mb, workloads, stream))

    cpu = cpu_baseline(wl, eff, args.cpu_seconds)
    if not args.no_extras:
        phase("cpu_baseline_all_cores", cpu_baseline_all_cores(wl, eff, args.cpu_seconds / 2))
        phase("cpu_baseline_python_small", cpu_baseline_python())

    traffic = counted_traffic()
    line = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {
            "workload": "mixed_bf16: in-place apply, bf16 logits [256,128256] N(0,2), vocab_size=128000, "
                        "mask int32 [256,4008] with per-row density U[0.001,0.5] and garbage padding words, "
                        "128 unique random row indices",
            "logits_dtype": "bfloat16",
            "rows_processed": R, "vocab_size": V, "variant": args.variant,
            "protocol": f"cold: {nsets} rotating buffer sets of {set_bytes / 1e6:.1f} MB, each launch touching "
                        f"{eff / 1e6:.1f} MB ({nsets * eff / 1e6:.0f} MB per cycle > 2 x 256 MB Infinity Cache); {args.steps} "
                        "launches captured in one HIP graph, timed by HIP events on the launch stream",
            "effective_bytes_per_step": eff,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_GBPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    if traffic is not None:
        # the same steps counted in the bytes that cross the HBM interface
        # (counters from the committed summary) rather than algorithmic bytes
        phys = traffic / (ms_step * 1e-3) / 1e9
        line["hbm_traffic_rate"] = {"bytes_per_step": traffic, "GBps": round(phys, 1),
                                    "frac_of_peak": round(phys / PEAK_GBPS, 4)}
    line.update(extras)
    print(json.dumps(line), flush=True)


def ceilings(torch, dev, eff, nsets, steps, stream, rmw_bytes=0):
    """Plain fill and copy over the same byte count, same rotation.

    With rmw_bytes, also a plain copy of rmw_bytes (read rmw_bytes, write
    rmw_bytes): the physical traffic of an in-place apply that must read
    every line it writes, without any of the apply's work.
    """
    n = eff // 2
    nsets = max(2, math.ceil(2 * INFINITY_CACHE / eff))
    bufs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(nsets)]
    half = [torch.empty(n // 2, dtype=torch.int16, device=dev) for _ in range(2 * nsets)]
    cases = [("fill", eff, lambda k: bufs[k % nsets].fill_(-128)),
             ("copy", eff, lambda k: half[(2 * k) % (2 * nsets)].copy_(half[(2 * k + 1) % (2 * nsets)]))]
    if rmw_bytes:
        rsets = max(2, math.ceil(INFINITY_CACHE / rmw_bytes))
        src = [torch.empty(rmw_bytes // 2, dtype=torch.int16, device=dev) for _ in range(rsets)]
        dst = [torch.empty(rmw_bytes // 2, dtype=torch.int16, device=dev) for _ in range(rsets)]
        cases.append(("copy_same_physical_bytes", 2 * rmw_bytes, lambda k: dst[k % rsets].copy_(src[k % rsets])))
    torch.cuda.synchronize()
    out = {}
    for name, nbytes, fn in cases:
        with torch.cuda.stream(stream):
            for k in range(10):
                fn(k)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for k in range(steps):
                fn(k)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / steps
        out[name] = {"bytes_per_step": nbytes, "ms_per_step": ms, "GBps": nbytes / (ms * 1e-3) / 1e9}
        del g
    return out


def own_copy(torch, dev, mb, rows, cols, mask_cols, steps, stream):
    """This library's out-of-place apply with an all-allowed mask over `rows` rows: a plain copy.

    It reads and writes every logit of those rows (and reads their mask
    words), the physical traffic of the in-place apply of a mask whose
    lines all mix kept and masked tokens, with the same load, store and
    launch machinery.  Cold rotation like the headline.
    """
    nbytes = 2 * rows * cols * 2 + rows * mask_cols * 4
    nsets = max(2, math.ceil(2 * INFINITY_CACHE / nbytes))
    sets = [(torch.empty(rows, cols, dtype=torch.bfloat16, device=dev).normal_(),
             torch.full((rows, mask_cols), -1, dtype=torch.int32, device=dev),
             torch.empty(rows, cols, dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    ms = graph_ms(torch, lambda k: mb.mi_apply_bitmask_out(sets[k % nsets][0], sets[k % nsets][1],
                                                           sets[k % nsets][2]), steps, stream)
    del sets
    torch.cuda.empty_cache()
    return {"bytes_per_step": nbytes, "ms_per_step": ms, "GBps": nbytes / (ms * 1e-3) / 1e9}


def graph_ms(torch, fn, steps, stream, warmup=10):
    with torch.cuda.stream(stream):
        for k in range(warmup):
            fn(k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for k in range(steps):
            fn(k)
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    with torch.cuda.stream(stream):
        g.replay()
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    del g
    return ms


def vocab_shard(torch, dev, mb, wl, steps, stream, shards=8):
    """One GPU's share of the headline under an 8-way vocabulary split.

    Shard 0 of the [256, 128256] bf16 logits: its own [256, 16032] buffer
    (16032 = 128256 / 8 = 501 mask words), the mask read in place through a
    strided view of the full [256, 4008] mask (row stride 4008 words), the
    same 128 indexed rows; cold rotation over buffer sets.
    """
    import numpy as np

    cols = wl.logits.shape[1] // shards
    words = cols // 32
    R = len(wl.indices)
    eff = effective_bytes(R, cols, 2)
    nsets = cold_sets(eff)  # 128 rows of the shard and their mask words per launch
    shard = np.ascontiguousarray(wl.logits[:, :cols])
    sets = [(torch.from_numpy(shard.view(np.int16)).to(dev).view(torch.bfloat16),
             torch.from_numpy(wl.mask).to(dev)[:, :words],
             torch.from_numpy(wl.indices).to(dev)) for _ in range(nsets)]
    ms = graph_ms(torch, lambda k: mb.mi_apply_bitmask_inplace(sets[k % nsets][0], sets[k % nsets][1], cols,
                                                               sets[k % nsets][2]), steps, stream)
    del sets
    torch.cuda.empty_cache()
    return {"workload": f"bf16 [256, {cols}] (vocab shard 0 of {shards}), mask view [256, {words}] with row stride "
                        f"{wl.mask.shape[1]} words, {R} indexed rows",
            "effective_bytes": eff, "ms_per_step": ms, "GBps": eff / (ms * 1e-3) / 1e9}


def gated_rows(torch, dev, mb, workloads, steps, stream):
    """Gated apply with the per-row report on the speculative-verify shape.

    fp16 logits [256 slots, 4 rows, 32000] applied in place with 80 % of the
    rows flagged, against the plain in-place apply given the same rows as an
    index list; both cold (rotating buffer sets).
    """
    import numpy as np

    wl = workloads.verify_fp16()
    rng = np.random.default_rng(6)
    gate = (rng.random(wl.rows) < 0.8).astype(np.int8)
    active = np.flatnonzero(gate).astype(np.int32)
    W = (wl.cols + 31) // 32
    eff = len(active) * (W * 4 + wl.cols * 2)
    nsets = cold_sets(eff)  # the flagged rows
    sets = [(torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.float16).view(256, 4, wl.cols),
             torch.from_numpy(wl.mask).to(dev)) for _ in range(nsets)]
    g = torch.from_numpy(gate).to(dev)
    idx = torch.from_numpy(active).to(dev)
    t_rep = graph_ms(torch, lambda k: mb.mi_apply_bitmask_rows(sets[k % nsets][0], sets[k % nsets][1], g,
                                                               report=True), steps, stream)
    t_gate = graph_ms(torch, lambda k: mb.mi_apply_bitmask_rows(sets[k % nsets][0], sets[k % nsets][1], g),
                      steps, stream)
    t_idx = graph_ms(torch, lambda k: mb.mi_apply_bitmask_inplace(sets[k % nsets][0], sets[k % nsets][1], None,
                                                                  idx), steps, stream)
    del sets
    torch.cuda.empty_cache()
    return {"workload": f"fp16 [256,4,32000] in place, {len(active)} of 1024 rows flagged",
            "effective_bytes": eff,
            "gated_with_report": {"ms_per_step": t_rep, "GBps": eff / (t_rep * 1e-3) / 1e9},
            "gated": {"ms_per_step": t_gate, "GBps": eff / (t_gate * 1e-3) / 1e9},
            "index_list_same_rows": {"ms_per_step": t_idx, "GBps": eff / (t_idx * 1e-3) / 1e9}}


def out_of_place_listed(torch, dev, mb, workloads, steps, stream):
    """Out of place with an index list on the speculative-verify shape.

    fp16 logits [1024, 32000] into a separate output, the mask applied to 128
    listed rows (random, unsorted) and every other row copied: one pass over
    every row (each block finds whether the list holds its row).  Effective
    bytes: every row read and written once, plus the listed rows' mask
    words.  Beside it, the same call with no list (every row masked) and a
    list of 1100 rows, past the one-pass limit of 1024 (a copy, then the
    in-place apply of the listed rows on the output).  Cold rotation.
    """
    import numpy as np

    wl = workloads.verify_fp16()
    rng = np.random.default_rng(9)
    W = (wl.cols + 31) // 32
    nsets = max(2, math.ceil(2 * INFINITY_CACHE / (2 * wl.logits.nbytes + wl.mask.nbytes)))
    sets = [(torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.float16), torch.from_numpy(wl.mask).to(dev),
             torch.empty(wl.rows, wl.cols, dtype=torch.float16, device=dev)) for _ in range(nsets)]
    out = {}
    for label, n in (("list_128", 128), ("no_list", None), ("list_1100_past_one_pass", 1100)):
        idx = None
        if n is not None:
            idx = torch.from_numpy(rng.choice(wl.rows, size=min(n, wl.rows), replace=False).astype(np.int32)).to(dev)
            if n > wl.rows:
                idx = torch.cat([idx, idx[: n - wl.rows]])
        listed = wl.rows if n is None else int(idx.numel())
        eff = wl.rows * wl.cols * 2 * 2 + min(listed, wl.rows) * W * 4
        ms = graph_ms(torch, lambda k: mb.mi_apply_bitmask_out(sets[k % nsets][0], sets[k % nsets][1],
                                                               sets[k % nsets][2], None, idx, -65504.0),
                      steps, stream)
        out[label] = {"ms_per_step": ms, "effective_bytes": eff, "GBps": eff / (ms * 1e-3) / 1e9}
    del sets
    torch.cuda.empty_cache()
    out["workload"] = "fp16 [1024,32000] out of place, fill -65504, verify_fp16 masks"
    return out


def upload_overlap(torch, dev, mb, wl, steps=30):
    """A decode step with the mask uploaded on the compute stream vs behind the forward.

    Per step: a bf16 GEMM [256, 8192] x [8192, 32000] stands in for the
    forward pass, the 256 x 4008 int32 mask (4.1 MB, already filled in pinned
    host memory) goes host -> device, and the apply runs on the GEMM's
    output.  "serial" copies the mask on the compute stream before the apply;
    "staged" uses MaskStager: the copy runs on a side stream while the GEMM
    runs.  Times are per step (HIP events on the compute stream).
    """
    import numpy as np

    B = 256
    a = torch.randn(B, 8192, device=dev, dtype=torch.bfloat16)
    w = torch.randn(8192, 32000, device=dev, dtype=torch.bfloat16)
    logits = torch.empty(B, 32000, device=dev, dtype=torch.bfloat16)
    host = torch.from_numpy(wl.mask).pin_memory()
    dmask = torch.empty_like(host, device=dev)
    stager = mb.MaskStager(B, 32 * wl.mask.shape[1], device=dev, depth=2)
    for _ in range(stager.depth):          # the grammar engine's host fill is not timed here
        stager.host().copy_(host)
    compute = torch.cuda.Stream()
    out = {}
    for mode in ("serial", "staged", "gemm_only"):
        for rep in range(2):   # first pass warms up
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record(compute)
            with torch.cuda.stream(compute):
                for _ in range(steps):
                    if mode == "staged":
                        stager.host()
                        stager.upload()
                    torch.mm(a, w, out=logits)
                    if mode == "serial":
                        dmask.copy_(host, non_blocking=True)
                        mb.mi_apply_bitmask_inplace(logits, dmask, 32000, None)
                    elif mode == "staged":
                        stager.apply_inplace(logits, 32000, None, stream=compute)
            e.record(compute)
            torch.cuda.synchronize()
        out[mode] = {"ms_per_step": s.elapsed_time(e) / steps}
    return {"what": "per decode step: bf16 GEMM [256,8192]x[8192,32000], 4.1 MB mask upload, apply",
            **out}


SAMPLER_MODES = (("greedy", dict(temperature=0.0)), ("unfiltered", dict(temperature=1.0)),
                 ("top_p_0.9", dict(top_p=0.9)), ("top_k_50", dict(top_k=50)),
                 ("top_k_50_top_p_0.9_min_p_0.05", dict(top_k=50, top_p=0.9, min_p=0.05)))


def sampler_times(torch, dev, mb, workloads, stream, steps=200):
    """The fused apply + sampler at the two batch/vocab shapes the logits-processor page times,
    the first of them with fp32 logits, and the first with sparse masks (each
    token allowed with probability 0.005, about 640 per row: the grammar
    masks of constrained decoding are often that sparse).

    Per launch: one token per row from the masked logits.  Bytes counted: one
    read of the logits of every row plus its mask words; the kernel reads the
    row once per pass (greedy 1, unfiltered 1; with top-k or top-p, 16-bit
    rows take 2 -- the key histogram and the draw -- or 1 when a short row is
    held in registers between them; fp32 rows take 2 -- the coarse 12-bit
    bucket pass, which also finds the maximum, and the draw that lists the
    cut's bucket).  The fp32 shape holds the bf16 shape's values widened.
    Cold: rotating buffer sets.  Calls take the binding's default workspace,
    so at B=1024 the modes with top-p hand out their dense rows first (a
    classifying launch, then the draw; both are timed); those modes are
    timed in row order too ("row_order_us_per_call", no workspace).
    """
    import numpy as np

    out = {}
    sparse = workloads.mixed_bf16(n_indices=0)
    rng = np.random.default_rng(17)
    sparse.mask[:] = workloads.pack_allowed(rng.random((sparse.rows, sparse.cols)) < 0.005, sparse.mask.shape[1], rng)
    for label, wl, fp32 in (("B256_V128000_bf16", workloads.mixed_bf16(n_indices=0), False),
                            ("B1024_V32000_fp16", workloads.verify_fp16(), False),
                            ("B256_V128000_fp32", workloads.mixed_bf16(n_indices=0), True),
                            ("B256_V128000_bf16_mask_density_0.005", sparse, False)):
        R, V = wl.rows, (wl.vocab_size or wl.cols)
        esize = 4 if fp32 else 2
        nbytes = R * V * esize + R * ((V + 31) // 32) * 4
        # the least a launch touches: every mask word of the rows and each
        # 128-byte line of logits that holds an allowed token (a sparse row's
        # filtered draw reads no other line); greedy and unfiltered rows read
        # more, so the rotation is cold for them too
        nsets = cold_sets(touched_lines(wl, esize))
        tdt = torch.bfloat16 if wl.dtype == "bfloat16" else torch.float16
        sets = []
        for _ in range(nsets):
            x = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(tdt)
            sets.append((x.float().contiguous() if fp32 else x, torch.from_numpy(wl.mask).to(dev)))
        tok = torch.empty(R, dtype=torch.int64, device=dev)
        res = {}
        for mode, kw in SAMPLER_MODES:
            ms = graph_ms(torch, lambda k, kw=kw: mb.mi_apply_bitmask_sample(
                sets[k % nsets][0], sets[k % nsets][1], wl.vocab_size, seed=1, offset=k, out=tok, **kw),
                steps, stream)
            res[mode] = {"us_per_call": ms * 1e3, "GBps_one_read": nbytes / (ms * 1e-3) / 1e9}
            if mb.sample_workspace_bytes(sets[0][0].dtype, R, V) > 0 and "top_p" in kw:
                ms0 = graph_ms(torch, lambda k, kw=kw: mb.mi_apply_bitmask_sample(
                    sets[k % nsets][0], sets[k % nsets][1], wl.vocab_size, seed=1, offset=k, out=tok, workspace=None,
                    **kw), steps, stream)
                res[mode]["row_order_us_per_call"] = ms0 * 1e3
            ref_ms = torch_sort_sampler_ms(torch, sets, wl.vocab_size or wl.cols, kw, stream)
            res[mode]["torch_sort_us_per_call"] = ref_ms * 1e3
            res[mode]["speedup_vs_torch_sort"] = ref_ms / ms
        out[label] = res
        del sets
        torch.cuda.empty_cache()
    return out


def touched_lines(wl, esize):
    """Mask bytes of every row plus 128 bytes per logits line holding an allowed token (tokens below V)."""
    import numpy as np

    V = wl.vocab_size or wl.cols
    bits = np.unpackbits(wl.mask.view(np.uint8), axis=1, bitorder="little")[:, :V].astype(bool)
    per_line = 128 // esize
    pad = (-V) % per_line
    lines = np.pad(bits, ((0, 0), (0, pad))).reshape(wl.rows, -1, per_line).any(axis=2).sum()
    return int(wl.mask.nbytes + lines * 128)


def sampler_small_batch(torch, dev, mb, workloads, stream, steps=200):
    """Every mode on the first B rows of the B=256 bf16 sampler shape, B = 1, 16, 32, 64.

    With few rows the library splits each row over several blocks: rows
    without a filter by themselves, filtered rows through a workspace (the
    default, up to 32 rows); these are the batch sizes where that matters.  The filtered
    modes are timed without the workspace too ("one_block_per_row").  The
    rows rotate over buffer sets sized for the full batch, but B rows of
    256 KB (at most 16.8 MB a set) stay in the caches across the rotation:
    these figures are cache-resident, as logits just written by the
    producing kernel would be, not HBM figures.
    """
    import numpy as np

    wl = workloads.mixed_bf16(n_indices=0)
    nsets = max(2, math.ceil(2 * INFINITY_CACHE / (wl.logits.nbytes + wl.mask.nbytes)))
    sets = [(torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16), torch.from_numpy(wl.mask).to(dev))
            for _ in range(nsets)]
    out = {}
    for B in (1, 16, 32, 64):
        tok = torch.empty(B, dtype=torch.int64, device=dev)
        res = {}
        for mode, kw in (("greedy", dict(temperature=0.0)), ("unfiltered", dict(temperature=1.0)),
                         ("top_k_50", dict(top_k=50)), ("top_p_0.9", dict(top_p=0.9)),
                         ("top_k_50_top_p_0.9_min_p_0.05", dict(top_k=50, top_p=0.9, min_p=0.05))):
            ms = graph_ms(torch, lambda k, kw=kw: mb.mi_apply_bitmask_sample(
                sets[k % nsets][0][:B], sets[k % nsets][1][:B], wl.vocab_size, seed=1, offset=k, out=tok, **kw),
                steps, stream)
            res[mode] = {"us_per_call": ms * 1e3}
            if mode.startswith("top"):
                ms1 = graph_ms(torch, lambda k, kw=kw: mb.mi_apply_bitmask_sample(
                    sets[k % nsets][0][:B], sets[k % nsets][1][:B], wl.vocab_size, seed=1, offset=k, out=tok,
                    workspace=None, **kw), steps, stream)
                res[mode]["one_block_per_row_us_per_call"] = ms1 * 1e3
        out[f"B{B}_V128000_bf16"] = res
    del sets
    torch.cuda.empty_cache()
    return out


def torch_sort_sampler_ms(torch, sets, V, kw, stream, steps=20):
    """The same draw done the usual way with stock torch ops, for comparison.

    Unpack the bitmask into a bool mask, fill the masked logits with -inf,
    then: greedy is an argmax; otherwise softmax of z = logit / T, and with
    top-k or top-p a descending sort, the filters on the sorted
    probabilities (top-k by rank, top-p on the exclusive cumulative sum,
    min-p against the largest) and torch.multinomial on what is left;
    unfiltered draws with torch.multinomial directly.  Rows with nothing
    allowed draw from a flat row (the fused kernel returns -1 for them).
    Eager launches on the same rotating buffer sets, timed by HIP events on
    the stream.
    """
    temperature = kw.get("temperature", 1.0)
    top_k, top_p, min_p = kw.get("top_k", 0), kw.get("top_p", 1.0), kw.get("min_p", 0.0)
    dev = sets[0][0].device
    tok_ids = torch.arange(V, device=dev)
    word, bit = tok_ids // 32, (tok_ids % 32).to(torch.int32)

    def one(k):
        logits, mask = sets[k % len(sets)]
        allowed = ((mask[:, word] >> bit) & 1).bool()
        x = logits[:, :V].float().masked_fill(~allowed, float("-inf"))
        # a row with nothing allowed would be all NaN after the softmax, which
        # multinomial rejects: draw such rows from a flat row instead
        x = torch.where(allowed.any(-1, keepdim=True), x, torch.zeros((), device=dev))
        if temperature <= 0:
            return x.argmax(-1)
        probs = torch.softmax(x / temperature, -1)
        if not (top_k or top_p < 1.0 or min_p):
            return torch.multinomial(probs, 1)
        sp, si = probs.sort(-1, descending=True)
        if top_k:
            sp[:, top_k:] = 0
        if top_p < 1.0:
            sp = sp.masked_fill(sp.cumsum(-1) - sp > top_p, 0)
        if min_p:
            sp = sp.masked_fill(sp < min_p * sp[:, :1], 0)
        return si.gather(1, torch.multinomial(sp, 1))

    with torch.cuda.stream(stream):
        for k in range(3):
            one(k)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for k in range(steps):
            one(k)
        e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def host_path(torch, mb, wl, eff, seconds=2.0):
    """The library's native host-memory apply (CPU tensors) on the same workload."""
    import numpy as np

    x = torch.from_numpy(wl.logits.copy().view(np.int16)).view(torch.bfloat16)
    m = torch.from_numpy(wl.mask)
    idx = list(wl.indices)
    passes, t0 = 0, time.perf_counter()
    while True:
        mb.mi_apply_bitmask_inplace_host(x, m, wl.vocab_size, idx)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max(1, (os.cpu_count() or 2) // 2)
    return {"GBps": eff * passes / el / 1e9, "passes": passes, "threads": threads,
            "note": "native C++ host entry point (not the oracle), default thread count"}


def cpu_baseline(wl, eff, seconds):
    """The oracle's C loop, one core, repeated full passes until `seconds` pass."""
    import oracle

    x = wl.logits.copy()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.apply_inplace(x, wl.mask, wl.dtype, wl.vocab_size, list(wl.indices), wl.fill_value)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(eff * passes / el / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full passes of the same workload (128 indexed rows x 128000 tokens) "
                      f"in {el:.1f} s on one host core"}


def cpu_baseline_all_cores(wl, eff, seconds):
    """The same oracle loop, the indexed rows split over the host's cores.

    One thread per core (at most 16), each applying its share of the rows
    again and again until `seconds` pass; the C loop releases the GIL, so
    the threads run in parallel.  Bytes per processed row are the
    workload's effective bytes over its rows.
    """
    import threading

    import numpy as np

    import oracle

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = [p for p in np.array_split(np.asarray(wl.indices), threads) if p.size]
    x = wl.logits.copy()
    done = [0] * len(parts)
    t0 = time.perf_counter()
    stop = t0 + seconds

    def work(k):
        rows = list(parts[k])
        while time.perf_counter() < stop:
            oracle.apply_inplace(x, wl.mask, wl.dtype, wl.vocab_size, rows, wl.fill_value)
            done[k] += len(rows)

    pool = [threading.Thread(target=work, args=(k,)) for k in range(len(parts))]
    for th in pool:
        th.start()
    for th in pool:
        th.join()
    el = time.perf_counter() - t0
    per_row = eff / len(wl.indices)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(sum(done) * per_row / el / 1e9, 3), "unit": "GB/s", "cores": len(parts),
            "kind": "oracle", "cpu_model": model,
            "sample": f"{sum(done)} row applications of the same workload's indexed rows, split over "
                      f"{len(parts)} threads, in {el:.1f} s"}


def cpu_baseline_python():
    """The oracle's pure-Python loop on the two small workloads, one pass each.

    The tiny fp32 [1, 32000] case and the bf16 [8, 50257] case with its
    garbage tail: the Python list version of the page's double loop, timed
    whole (conversion to and from lists included).
    """
    import oracle
    import workloads

    out = {}
    for wl in (workloads.tiny(), workloads.tail_bf16()):
        rows, cols = wl.logits.shape
        V = wl.vocab_size if wl.vocab_size is not None else min(cols, 32 * wl.mask.shape[1])
        eff = effective_bytes(rows, V, wl.logits.dtype.itemsize)
        t0 = time.perf_counter()
        oracle.apply_inplace_py(wl.logits, wl.mask, wl.dtype, wl.vocab_size, None, wl.fill_value)
        el = time.perf_counter() - t0
        out[wl.name] = {"seconds": round(el, 3), "GBps": round(eff / el / 1e9, 5), "cores": 1}
    return out


if __name__ == "__main__":
    main()
