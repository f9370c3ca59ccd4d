"""Benchmark of the PlaneZip hot path on one MI355X.

One step = compress and then decompress every tensor of the workload (the
GPT-2-XL activations at batch 8, sequence 1024: MLP GELU output 8x1024x6400,
causal softmax 8x25x1024x1024, residual 8x1024x1600, all BF16, ~0.55 GB),
each tensor into and out of its own stream, on one HIP stream, with inputs
already resident in HBM: one pz_compress_batch call and then one
pz_decompress_batch call over the tensors (one launch per kernel). The same
step made of one pz_compress / pz_decompress call per tensor is timed as well
(`per_call`, and the per-tensor rates). Before every step (warm-up and timed)
a 1 GiB buffer is written, outside the timed region, so that no step finds
its inputs in the 256 MB last-level cache (MALL); each timed step is
bracketed by device synchronizations and timed with HIP events recorded
behind the flush (so the host has enqueued the step before the GPU starts
it). Prints one JSON line.

value = raw bytes of the workload / mean time of one step (each raw byte is
both compressed and decompressed in a step). The roofline object reports the
dominant kernel's algorithmic HBM traffic (raw plus compressed bytes, one
read and the other written) per unit of its measured time against MI355X's
8 TB/s: the longer of the batched compress launch and, when it is a single
kernel, the batched decompress launch. The CPU baseline is the
oracle (oracle/pzref.c) on the same tensors on this host's cores: chunk-
parallel on the whole workload, and single-threaded on a bounded sample.

Outside the timed regions the line also carries, per tensor, the encoder mix
(blocks won by each candidate, the most frequent one, chunks stored raw: the
'Top' column of the paper's Table III), the other four workloads' batched
compress and decompress rates, HBM fractions and ratios (`workloads`), and a
byte-for-byte comparison of every GPU stream with the oracle's stream of the
same tensor (`oracle_equal`, made in the CPU-baseline leg).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="gpt2-xl", choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--cpu-sample-mb", type=float, default=24.0,
                   help="sample of the workload for the single-threaded oracle timing")
    p.add_argument("--no-flush", action="store_true", help="skip the cache flush before each step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-verify", action="store_true")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (HBM counter calibration)")
    p.add_argument("--no-swap", action="store_true", help="skip the copy-path (swap) measurement")
    p.add_argument("--headline-only", action="store_true",
                   help="skip the rates, ratios and oracle checks of the other workloads")
    p.add_argument("--variants", action="store_true",
                   help="also time the codec variants the paper compares PlaneZip with (Fig. 3) "
                        "on the same tensors and report their ratios")
    return p.parse_args()


# The synthetic workloads (pzinputs), by what they stand in for.
WORKLOADS = {
    "relu-smoke": "codec smoke tensor: ReLU(N(0,1)) BF16, 1 MiB, plus 64 corner-case blocks",
    "cnn-fp32": "CNN feature maps, FP32 NCHW 32x64x56x56, ReLU of smoothed noise",
    "gpt2-small": "GPT-2 (124M) BF16 saved activations, batch 8, seq 1024: MLP GELU 8x1024x3072, "
                  "causal attention probabilities 8x12x1024x1024",
    "vit-layernorm": "ViT-B/16 LayerNorm outputs 64x197x768, BF16 and FP32",
    "gpt2-xl": "GPT-2-XL BF16 saved activations, batch 8, seq 1024: MLP GELU 8x1024x6400, "
               "causal softmax 8x25x1024x1024, residual 8x1024x1600",
}
WORKLOAD_NAMES = tuple(WORKLOADS)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}). The codec would shard a "
              "tensor into contiguous chunk ranges, one per GPU, with one exclusive scan of the "
              "per-shard stream sizes; only the single-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import lossless_bit_plane_amd as pz
    import pzinputs

    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del a, b
    t0 = time.time()
    tensors = pzinputs.workload(args.workload)
    log(f"generated workload {args.workload} in {time.time() - t0:.1f}s: "
        + ", ".join(f"{t.name} {t.nbytes / 1e6:.1f} MB" for t in tensors))
    inputs_ok = input_check(args.workload, tensors)
    log(f"inputs against the SHA-256 manifest: {inputs_ok}")

    # Device buffers, allocated once.
    items = []
    for t in tensors:
        src = torch.from_numpy(t.data).to(dev)
        cap = pz.max_compressed_bytes(t.nbytes)
        items.append(dict(
            t=t, src=src,
            stream=torch.empty(cap, dtype=torch.uint8, device=dev),
            nbytes=torch.zeros(1, dtype=torch.int64, device=dev),
            out=torch.empty(t.nbytes, dtype=torch.uint8, device=dev),
            status=torch.zeros(1, dtype=torch.int32, device=dev),
        ))
    torch.cuda.synchronize()

    # Compressed sizes (device-side, read once before timing).
    for it in items:
        pz.pz_compress(it["src"], it["t"].dtype, it["t"].elem_bits, it["stream"], it["nbytes"])
    torch.cuda.synchronize()
    for it in items:
        it["comp"] = int(it["nbytes"].item())

    cur = torch.cuda.current_stream()
    flush_buf = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def flush():
        if flush_buf is not None:
            flush_buf.fill_(0x5A)

    copy_gbps = measure_copy(torch, dev, cur)
    log(f"plain device copy of 512 MiB: {copy_gbps:.0f} GB/s of reads plus writes")

    # Batched step: one call per direction for each (dtype, width) group of
    # tensors (the bench workload is one group).
    groups = {}
    for it in items:
        groups.setdefault((it["t"].dtype, it["t"].elem_bits), []).append(it)
    for (dt, w), g in groups.items():
        g[0]["group_out"] = torch.zeros(len(g), dtype=torch.int64, device=dev)
        g[0]["group_status"] = torch.zeros(len(g), dtype=torch.int32, device=dev)

    def step(events=None):
        if events is not None:
            events[0].record(cur)
        for (dt, w), g in groups.items():
            pz.pz_compress_batch([it["src"] for it in g], dt, w, [it["stream"] for it in g], g[0]["group_out"])
        if events is not None:
            events[1].record(cur)
        for (dt, w), g in groups.items():
            pz.pz_decompress_batch([it["stream"] for it in g], [it["comp"] for it in g],
                                   [it["t"].nbytes for it in g], dt, w, [it["out"] for it in g],
                                   g[0]["group_status"])
        if events is not None:
            events[2].record(cur)

    def step_calls(events=None):
        for i, it in enumerate(items):
            t = it["t"]
            if events is not None:
                events[i][0].record(cur)
            pz.pz_compress(it["src"], t.dtype, t.elem_bits, it["stream"], it["nbytes"])
            if events is not None:
                events[i][1].record(cur)
        for i, it in enumerate(items):
            t = it["t"]
            if events is not None:
                events[i][2].record(cur)
            pz.pz_decompress(it["stream"], it["comp"], t.nbytes, t.dtype, t.elem_bits,
                             it["out"], it["status"])
            if events is not None:
                events[i][3].record(cur)

    def verify(what):
        for it in items:
            assert int(it["status"].item()) == 0, f"{what}: decompress reported a corrupt stream"
            assert torch.equal(it["out"], it["src"]), f"{what}: round trip mismatch on {it['t'].name}"
        for g in groups.values():
            assert not g[0]["group_status"].any().item(), f"{what}: decompress reported a corrupt stream"
            assert [int(v) for v in g[0]["group_out"].tolist()] == [it["comp"] for it in g], what
        log(f"{what}: round trip verified on the device")

    for _ in range(args.warmup):
        flush()
        step_calls()
        flush()
        step()
    torch.cuda.synchronize()
    if not args.no_verify:
        verify("warm-up")

    def timed_steps(fn, nev):
        # Each step sits between two device synchronizations. The cache flush
        # is enqueued first and the step's start event behind it, so the
        # host has enqueued the whole step by the time the GPU reaches it
        # (the events time the GPU's work, not the host's submission).
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
        step_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        enqueue = 0.0
        for k in range(args.steps):
            torch.cuda.synchronize()
            flush()
            start = time.perf_counter()
            step_ev[k][0].record(cur)
            fn(ev[k])
            step_ev[k][1].record(cur)
            enqueue += time.perf_counter() - start
            torch.cuda.synchronize()
        return ev, np.array([a.elapsed_time(b) for a, b in step_ev]), enqueue

    # One pz_compress / pz_decompress call per tensor: per-tensor rates.
    ev_c, step_ms_c, _ = timed_steps(
        lambda e: step_calls([[e[4 * i + j] for j in range(4)] for i in range(len(items))]), 4 * len(items))
    # The batched step: the bench line.
    ev, step_ms, wall = timed_steps(step, 3)
    if not args.no_verify:
        verify("timed steps")

    raw_total = sum(it["t"].nbytes for it in items)
    comp_total = sum(it["comp"] for it in items)
    t_comp = np.zeros(len(items))
    t_dec = np.zeros(len(items))
    for k in range(args.steps):
        for i in range(len(items)):
            t_comp[i] += ev_c[k][4 * i].elapsed_time(ev_c[k][4 * i + 1]) / 1e3
            t_dec[i] += ev_c[k][4 * i + 2].elapsed_time(ev_c[k][4 * i + 3]) / 1e3
    t_comp /= args.steps
    t_dec /= args.steps
    ms_per_step = float(step_ms.mean())
    value = raw_total / (ms_per_step / 1e3) / 1e9

    comp_s = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) / 1e3
    dec_s = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) / 1e3
    algo = raw_total + comp_total  # algorithmic HBM bytes per direction
    comp_gbps = algo / comp_s / 1e9
    dec_gbps = algo / dec_s / 1e9
    # The dominant kernel: a pz_compress_batch call is one launch of
    # compress_kernel over the group's tensors (it reads R and writes C); a
    # pz_decompress_batch call of at least SINGLE_LAUNCH_MIN_TILES locate
    # tiles is one launch of decompress_kernel (it reads C and writes R).
    # The roofline reports the longer of the two.
    single = all(sum(locate_tiles(it["t"].nbytes) for it in g) >= SINGLE_LAUNCH_MIN_TILES
                 for g in groups.values())
    launches = [batch_name([it["t"].name for it in g]) for g in groups.values()]
    if single and dec_s > comp_s:
        kernel, gbps = "decompress_kernel", dec_gbps
        desc = "decompress_kernel (one pz_decompress_batch launch over the workload's tensors: locate and decode)"
    else:
        kernel, gbps = "compress_kernel<16>", comp_gbps
        desc = "compress_kernel (one pz_compress_batch launch over the workload's tensors)"
    traffic, traffic_note = measured_traffic(kernel, launches)
    roofline = {
        "bound": "hbm",
        "kernel": desc,
        "achieved": round(gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(gbps / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes": algo,
        "traffic_note": traffic_note,
        # A plain device-to-device copy in the same run: what the memory
        # system gives a kernel with nothing to compute (reads plus writes).
        "copy_gbps": round(copy_gbps, 1),
        "frac_of_copy": round(gbps / copy_gbps, 4),
    }

    p10, p50, p90 = (float(x) for x in np.percentile(step_ms, [10, 50, 90]))

    per_tensor = {it["t"].name: {
        "raw_bytes": it["t"].nbytes, "compressed_bytes": it["comp"],
        "ratio": round(it["t"].nbytes / it["comp"], 4),
        "compress_raw_gbps": round(it["t"].nbytes / t_comp[i] / 1e9, 1),
        "decompress_raw_gbps": round(it["t"].nbytes / t_dec[i] / 1e9, 1),
        **block_stats(pz, it),
        "input_sha256_ok": inputs_ok[it["t"].name],
    } for i, it in enumerate(items)}
    # The GPU streams, on the host, for the byte-for-byte check against the
    # oracle's streams (outside every timed region).
    gpu_streams = {it["t"].name: it["stream"][:it["comp"]].cpu().numpy() for it in items}

    # The other workloads: batched compress and decompress rates, ratios and
    # block statistics (their streams are checked against the oracle below).
    workloads = {}
    other_streams = {}
    if not args.headline_only:
        for name in WORKLOAD_NAMES:
            if name != args.workload:
                workloads[name], other_streams[name] = measure_workload(pz, pzinputs, name, flush, cur)

    cpu = None
    oracle_equal = None
    if not args.no_cpu_baseline:
        cpu, oracle_equal = cpu_baseline(tensors, args.cpu_sample_mb, gpu_streams)
        for name, (tens, streams) in other_streams.items():
            eq, rates = oracle_check(tens, streams)
            workloads[name]["oracle_equal"] = all(eq.values())
            workloads[name]["cpu_oracle"] = rates
            for tname, ok in eq.items():
                workloads[name]["tensors"][tname]["oracle_equal"] = ok
        for tname, ok in oracle_equal.items():
            per_tensor[tname]["oracle_equal"] = ok
        if not all(oracle_equal.values()) or not all(c["oracle_equal"] for c in workloads.values()):
            log("GPU stream differs from the oracle's stream")
    other_streams.clear()

    variants = measure_variants(pz, items, flush, cur) if args.variants else None
    size_only = measure_size_only(pz, items, flush, cur)
    swap = None if args.no_swap else measure_swap(pz, items, flush)
    if swap is not None:
        swap["eq2"] = eq2_prediction(pz, items, per_tensor, swap)

    ms_calls = float(step_ms_c.mean())
    per_call = {
        "ms_per_step": round(ms_calls, 4),
        "value": round(raw_total / (ms_calls / 1e3) / 1e9, 2),
        "compress_raw_gbps": round(raw_total / t_comp.sum() / 1e9, 1),
        "decompress_raw_gbps": round(raw_total / t_dec.sum() / 1e9, 1),
        "step_ms_median": round(float(np.median(step_ms_c)), 4),
    }

    out = {
        "metric": "compress & decompress GB/s (raw bytes), % of HBM roofline; ratio = oracle",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ", ".join(sorted({f"u{t.elem_bits} symbols" for t in tensors})) + ", integer codec",
        "data": "synthetic (seeded generators in pzinputs, stand-ins for captured activations)",
        "config": {
            "workload": WORKLOADS[args.workload],
            "tensors": [f"{t.name} {list(t.shape)}" for t in tensors],
            "raw_bytes": raw_total,
            "compressed_bytes": comp_total,
            "ratio": round(raw_total / comp_total, 4),
            "parallelism": "single GPU",
            "calls": "pz_compress_batch then pz_decompress_batch over the tensors (separate streams, "
                     "one launch per kernel); per_call: one call per tensor and direction",
        },
        "step_ms": {"median": round(p50, 4), "p10": round(p10, 4), "p90": round(p90, 4),
                    "host_enqueue_ms_mean": round(wall / args.steps * 1e3, 4),
                    "cache_flush_before_each_step": flush_buf is not None},
        "compress_raw_gbps": round(raw_total / comp_s / 1e9, 1),
        "decompress_raw_gbps": round(raw_total / dec_s / 1e9, 1),
        "compress_hbm_frac": round(comp_gbps / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "per_call": per_call,
        "cpu_baseline": cpu,
        "oracle_equal": None if oracle_equal is None else (
            all(oracle_equal.values()) and all(c["oracle_equal"] for c in workloads.values())),
        "tensors": per_tensor,
        "workloads": workloads,
        "size_only": size_only,
        "swap": swap,
    }
    if variants is not None:
        out["variants"] = variants
    print(json.dumps(out), flush=True)


def measure_copy(torch, dev, cur, nbytes=512 << 20, reps=5):
    """Read-plus-write GB/s of a plain device-to-device copy (torch's copy
    kernel), best of `reps`, HIP events on the current stream."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    best = float("inf")
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(cur)
        b.copy_(a)
        e[1].record(cur)
        torch.cuda.synchronize()
        best = min(best, e[0].elapsed_time(e[1]) / 1e3)
    del a, b
    return 2 * nbytes / best / 1e9


TAG_NAMES = ("ZVC", "DBX", "BX", "ZBX", "RAW")  # tags 0..4
MANIFEST = os.path.join(ROOT, "tests", "golden", "input_sha256.txt")


def input_check(workload, tensors):
    """SHA-256 of each input tensor against the committed manifest
    (tests/golden/input_sha256.txt): True / False by tensor name, None for a
    tensor the manifest does not list."""
    known = {}
    if os.path.exists(MANIFEST):
        with open(MANIFEST) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    w, name, nbytes, digest = line.split()
                    known[(w, name)] = (int(nbytes), digest)
    out = {}
    for t in tensors:
        k = known.get((workload, t.name))
        out[t.name] = None if k is None else (k[0] == t.nbytes and k[1] == t.sha256())
    return out


def block_stats(pz, it):
    """A tensor's encoder mix (the 'Top' column of PlaneZip's Table III):
    the blocks each candidate wins (pz_block_sizes, the compressor's own
    choice per block), the most frequent one, and the chunks stored raw
    (header value equal to the chunk's length)."""
    import torch

    t = it["t"]
    _, tags = pz.pz_block_sizes(it["src"], t.dtype, t.elem_bits)
    hist = torch.bincount(tags.long(), minlength=5)[:5].tolist()
    C = pz.num_chunks(t.nbytes)
    H = it["stream"][:2 * C].view(torch.int16).to(torch.int32) & 0xFFFF
    raw_len = torch.full((C,), 4096, dtype=torch.int32, device=H.device)
    raw_len[-1] = t.nbytes - 4096 * (C - 1)
    raw_chunks = int((H == raw_len).sum().item())
    total = max(1, sum(hist))
    return {
        "block_tags": {n: int(c) for n, c in zip(TAG_NAMES, hist)},
        "block_tag_share": {n: round(c / total, 4) for n, c in zip(TAG_NAMES, hist)},
        "top": TAG_NAMES[int(np.argmax(hist))],
        "chunks": C,
        "raw_chunks": raw_chunks,
    }


def measure_workload(pz, pzinputs, name, flush, cur, reps=20, warmup=3):
    """One workload's batched compress and decompress (one call per
    direction and (dtype, width) group, as in the headline step): raw GB/s
    and fraction of HBM peak of the algorithmic bytes (read raw + write
    stream, or the reverse), median of `reps` after a cache flush each; the
    ratio and block statistics per tensor; round trip checked on the device.
    Returns (result, (tensors, host copies of the GPU streams))."""
    import torch

    dev = torch.device("cuda:0")
    tensors = pzinputs.workload(name)
    inputs_ok = input_check(name, tensors)
    items = []
    for t in tensors:
        items.append(dict(t=t, src=torch.from_numpy(t.data).to(dev),
                          stream=torch.empty(max(16, pz.max_compressed_bytes(t.nbytes)), dtype=torch.uint8,
                                             device=dev),
                          out=torch.empty(max(16, t.nbytes), dtype=torch.uint8, device=dev)))
    groups = {}
    for it in items:
        groups.setdefault((it["t"].dtype, it["t"].elem_bits), []).append(it)
    outs = {k: torch.zeros(len(g), dtype=torch.int64, device=dev) for k, g in groups.items()}
    stats = {k: torch.zeros(len(g), dtype=torch.int32, device=dev) for k, g in groups.items()}
    for k, g in groups.items():
        pz.pz_compress_batch([it["src"] for it in g], k[0], k[1], [it["stream"] for it in g], outs[k])
    torch.cuda.synchronize()
    for k, g in groups.items():
        for it, m in zip(g, outs[k].tolist()):
            it["comp"] = int(m)

    def compress():
        for k, g in groups.items():
            pz.pz_compress_batch([it["src"] for it in g], k[0], k[1], [it["stream"] for it in g], outs[k])

    def decompress():
        for k, g in groups.items():
            pz.pz_decompress_batch([it["stream"] for it in g], [it["comp"] for it in g],
                                   [it["t"].nbytes for it in g], k[0], k[1], [it["out"] for it in g], stats[k])

    def timed(fn):
        for _ in range(warmup):
            fn()
        ts = []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            torch.cuda.synchronize()
            flush()
            e[0].record(cur)
            fn()
            e[1].record(cur)
            torch.cuda.synchronize()
            ts.append(e[0].elapsed_time(e[1]) / 1e3)
        return np.array(ts)

    ts_c, ts_d = timed(compress), timed(decompress)
    t_c, t_d = float(np.median(ts_c)), float(np.median(ts_d))
    for k, g in groups.items():
        assert [int(v) for v in outs[k].tolist()] == [it["comp"] for it in g], f"{name}: unstable stream length"
        assert not stats[k].any().item(), f"{name}: decompress reported a corrupt stream"
        for it in g:
            assert torch.equal(it["out"][:it["t"].nbytes], it["src"]), f"{name}: round trip on {it['t'].name}"
    raw = sum(it["t"].nbytes for it in items)
    comp = sum(it["comp"] for it in items)
    res = {
        "workload": WORKLOADS[name],
        "raw_bytes": raw, "compressed_bytes": comp, "ratio": round(raw / comp, 4),
        "compress_raw_gbps": round(raw / t_c / 1e9, 1),
        "decompress_raw_gbps": round(raw / t_d / 1e9, 1),
        "compress_hbm_frac": round((raw + comp) / t_c / 1e9 / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round((raw + comp) / t_d / 1e9 / HBM_PEAK_GBPS, 4),
        "us": {d: {"median": round(float(np.median(v)) * 1e6, 1), "p10": round(float(np.percentile(v, 10)) * 1e6, 1),
                   "p90": round(float(np.percentile(v, 90)) * 1e6, 1)}
               for d, v in (("compress", ts_c), ("decompress", ts_d))},
        "timing": f"HIP events around each call, {warmup} warm-up calls, {reps} timed, a cache flush before each",
        "launches": f"{len(groups)} pz_compress_batch + {len(groups)} pz_decompress_batch call(s)",
        "tensors": {it["t"].name: {"raw_bytes": it["t"].nbytes, "compressed_bytes": it["comp"],
                                   "ratio": round(it["t"].nbytes / it["comp"], 4), **block_stats(pz, it),
                                   "input_sha256_ok": inputs_ok[it["t"].name]}
                    for it in items},
        "oracle_equal": None,
    }
    log(f"workload {name}: ratio {raw / comp:.3f}, compress {raw / t_c / 1e9:.0f} GB/s, "
        f"decompress {raw / t_d / 1e9:.0f} GB/s")
    streams = {it["t"].name: it["stream"][:it["comp"]].cpu().numpy() for it in items}
    del items
    torch.cuda.empty_cache()
    return res, (tensors, streams)


# The codecs of the paper's comparison (§V-A, Fig. 3) that are defined on the
# pages, as (candidate mask, tagged, symbol width or None for the tensor's):
# ZVC alone as in cDMA, BPC's DBX on every block, BX and ZBX alone, PlaneZip,
# and PlaneZip on BF16 coded as 32-bit symbols (the width BPC itself uses).
VARIANTS = {
    "ZVC": (0x01, False, None),
    "BPC (DBX on every block)": (0x02, False, None),
    "BX": (0x04, False, None),
    "ZBX": (0x08, False, None),
    "PlaneZip": (0x1F, True, None),
    "PlaneZip, 32-bit symbols": (0x1F, True, 32),
}


def measure_variants(pz, items, flush, cur, reps=3):
    """Ratio and raw GB/s of every variant on the workload's tensors (median
    of `reps` timed compress and decompress calls per tensor, each after a
    cache flush), round trip checked."""
    import torch

    res = {}
    for name, (mask, tagged, w) in VARIANTS.items():
        raw = comp = 0
        tc = td = 0.0
        per = {}
        for it in items:
            t = it["t"]
            bits = w or t.elem_bits
            cs, ds = [], []
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                flush()
                e[0].record(cur)
                pz.pz_compress_ex(it["src"], mask, tagged, t.dtype, bits, it["stream"], it["nbytes"])
                e[1].record(cur)
                torch.cuda.synchronize()
                n = int(it["nbytes"].item())
                flush()
                e[2].record(cur)
                pz.pz_decompress_ex(it["stream"], n, t.nbytes, t.dtype, bits, mask, tagged,
                                    it["out"], it["status"])
                e[3].record(cur)
                torch.cuda.synchronize()
                assert int(it["status"].item()) == 0 and torch.equal(it["out"], it["src"]), name
                cs.append(e[0].elapsed_time(e[1]) / 1e3)
                ds.append(e[2].elapsed_time(e[3]) / 1e3)
            c, d = float(np.median(cs)), float(np.median(ds))
            raw += t.nbytes
            comp += n
            tc += c
            td += d
            per[t.name] = round(t.nbytes / n, 4)
        res[name] = {"ratio": round(raw / comp, 4), "ratio_per_tensor": per,
                     "compress_raw_gbps": round(raw / tc / 1e9, 1),
                     "decompress_raw_gbps": round(raw / td / 1e9, 1)}
        log(f"variant {name}: ratio {raw / comp:.3f}, compress {raw / tc / 1e9:.0f} GB/s, "
            f"decompress {raw / td / 1e9:.0f} GB/s")
    return res


def measure_size_only(pz, items, flush, cur, stride=4, reps=5):
    """The runtime's size measurements on the workload (PlaneZip §III-B: a
    profiling iteration sizes tensors without keeping a stream): the exact
    size pass and the sampled one over every `stride`-th chunk, as raw GB/s
    (median of `reps` calls per tensor, each after a cache flush), with the
    sampled estimate's error against the exact size."""
    import torch

    sample = torch.zeros(2, dtype=torch.int64, device=items[0]["src"].device)
    res = {}
    for name in ("exact", "sampled"):
        raw = comp = est = 0
        t_total = 0.0
        for it in items:
            t = it["t"]
            ts = []
            for _ in range(reps):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                flush()
                e[0].record(cur)
                if name == "exact":
                    pz.pz_compressed_size(it["src"], t.dtype, t.elem_bits)
                else:
                    out, _ = pz.pz_compressed_size_sampled(it["src"], stride, t.dtype, t.elem_bits)
                e[1].record(cur)
                torch.cuda.synchronize()
                ts.append(e[0].elapsed_time(e[1]) / 1e3)
            if name == "exact":
                n, _ = pz.pz_compressed_size(it["src"], t.dtype, t.elem_bits)
                size = int(n.item())
                assert size == it["comp"], "size pass disagrees with the stream length"
            else:
                s_comp, s_raw = (int(v) for v in out.cpu().tolist())
                size = t.nbytes * s_comp / s_raw
            raw += t.nbytes
            comp += it["comp"]
            est += size
            t_total += float(np.median(ts))
        res[name] = {"raw_gbps": round(raw / t_total / 1e9, 1), "us": round(t_total * 1e6, 1)}
        if name == "sampled":
            res[name].update(stride=stride, estimate_bytes=round(est), exact_bytes=comp,
                             estimate_err_pct=round(100 * (est - comp) / comp, 4))
        log(f"size pass {name}: {raw / t_total / 1e9:.0f} GB/s ({t_total * 1e6:.0f} us)")
    # The exact sizes of every tensor in one pz_compressed_size_batch call per
    # (dtype, width) group.
    groups = {}
    for it in items:
        groups.setdefault((it["t"].dtype, it["t"].elem_bits), []).append(it)
    ts = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        flush()
        e[0].record(cur)
        outs = [pz.pz_compressed_size_batch([it["src"] for it in g], dt, w)[0] for (dt, w), g in groups.items()]
        e[1].record(cur)
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]) / 1e3)
    for out, g in zip(outs, groups.values()):
        assert [int(v) for v in out.tolist()] == [it["comp"] for it in g], "batched size pass disagrees"
    raw = sum(it["t"].nbytes for it in items)
    t_b = float(np.median(ts))
    res["exact_batched"] = {"raw_gbps": round(raw / t_b / 1e9, 1), "us": round(t_b * 1e6, 1)}
    log(f"size pass exact, batched: {raw / t_b / 1e9:.0f} GB/s ({t_b * 1e6:.0f} us)")
    return res


def measure_swap(pz, items, flush, reps=3, pool_chunk_bytes=2 << 20):
    """The copy path (PlaneZip §III, Fig. 2) on the workload, against plain
    copies of the raw tensors between HBM and pinned host memory. Swap-out:
    every tensor compressed into a staging slot and its stream copied into the
    pinned pool (the engine's worker issues the copies once each length is
    known); swap-in: the streams copied back and decompressed. Each figure is
    the workload's raw bytes over the host wall-clock time from the first
    call to the last completion (median of `reps`, each after a cache flush),
    round trip checked."""
    import torch

    raw_total = sum(it["t"].nbytes for it in items)
    comp_total = sum(it["comp"] for it in items)
    cur = torch.cuda.current_stream()

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    hosts = [torch.empty(it["t"].nbytes, dtype=torch.uint8, pin_memory=True) for it in items]

    def d2h():
        for h, it in zip(hosts, items):
            h.copy_(it["src"], non_blocking=True)
        torch.cuda.synchronize()

    def h2d():
        for h, it in zip(hosts, items):
            it["out"].copy_(h, non_blocking=True)
        torch.cuda.synchronize()

    t_d2h, t_h2d = timed(d2h), timed(h2d)
    for it in items:
        assert torch.equal(it["out"], it["src"]), "plain copy round trip"
    del hosts

    staging = max(pz.max_compressed_bytes(it["t"].nbytes) for it in items)
    chunks = sum(-(-it["comp"] // pool_chunk_bytes) for it in items) + 8
    sw = pz.Swapper(pool_chunk_bytes, chunks, staging, 2)
    tickets = []
    try:
        def swap_out():
            tickets.clear()
            for it in items:
                t = it["t"]
                tickets.append(sw.swap_out(it["src"], t.dtype, t.elem_bits))
            for k in tickets:
                sw.wait(k)

        def swap_in():
            for k, it in zip(tickets, items):
                sw.swap_in(k, it["out"], it["status"], cur)
            torch.cuda.synchronize()

        outs, ins = [], []
        for _ in range(reps):
            outs.append(timed_once(swap_out, flush))
            for k, it in zip(tickets, items):
                assert sw.wait(k) == it["comp"], "pool stream length"
            ins.append(timed_once(swap_in, flush))
            for it in items:
                assert int(it["status"].item()) == 0 and torch.equal(it["out"], it["src"]), "swap round trip"
            for k in tickets:
                sw.release(k)
        t_out, t_in = float(np.median(outs)), float(np.median(ins))
    finally:
        sw.close()
    res = {
        "raw_bytes": raw_total, "stream_bytes": comp_total, "pool_chunk_bytes": pool_chunk_bytes,
        "plain_d2h_gbps": round(raw_total / t_d2h / 1e9, 2),
        "plain_h2d_gbps": round(raw_total / t_h2d / 1e9, 2),
        "swap_out_gbps": round(raw_total / t_out / 1e9, 2),
        "swap_in_gbps": round(raw_total / t_in / 1e9, 2),
        "swap_out_speedup": round(t_d2h / t_out, 3),
        "swap_in_speedup": round(t_h2d / t_in, 3),
        "ms": {"plain_d2h": round(t_d2h * 1e3, 3), "plain_h2d": round(t_h2d * 1e3, 3),
               "swap_out": round(t_out * 1e3, 3), "swap_in": round(t_in * 1e3, 3)},
    }
    log(f"swap: plain D2H {res['plain_d2h_gbps']} GB/s, swap-out {res['swap_out_gbps']} GB/s "
        f"(x{res['swap_out_speedup']}); plain H2D {res['plain_h2d_gbps']} GB/s, swap-in "
        f"{res['swap_in_gbps']} GB/s (x{res['swap_in_speedup']})")
    return res


def eq2_prediction(pz, items, per_tensor, swap):
    """The planner's cost model (§III-C, Eq. 2) fed with this run's
    measurements: for each tensor x_t = min(m/g, max(m/(c g), m/B)), with g the
    measured plain pinned-copy rate of each direction, B the tensor's measured
    compress (decompress) rate and c its ratio; summed over the workload and set
    beside the measured swap-out (swap-in) time."""
    res = {}
    for d, link, rate, measured in (("out", swap["plain_d2h_gbps"], "compress_raw_gbps", swap["ms"]["swap_out"]),
                                    ("in", swap["plain_h2d_gbps"], "decompress_raw_gbps", swap["ms"]["swap_in"])):
        x = sum(pz.transfer_time(it["t"].nbytes, it["t"].nbytes / it["comp"], link * 1e9,
                                 per_tensor[it["t"].name][rate] * 1e9) for it in items)
        res[f"swap_{d}_predicted_ms"] = round(x * 1e3, 3)
        res[f"swap_{d}_measured_ms"] = measured
    return res


def timed_once(fn, flush):
    import torch

    flush()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


# Decompression of a launch of at least this many locate tiles (counted in
# tiles of 64 chunks) is one kernel, decompress_kernel; below it,
# locate_kernel and then decode_kernel (the library's threshold,
# pz_decompress.hip).
SINGLE_LAUNCH_MIN_TILES = 512


def locate_tiles(raw_bytes):
    chunks = (raw_bytes + 4095) // 4096
    return (chunks + 63) // 64


# The sources each kernel is built from: counters taken for a kernel stay
# valid while these files are unchanged.
KERNEL_SOURCES = {
    "compress_kernel": ["pz_device.h", "pz_compress.hip"],
    "locate_kernel": ["pz_device.h", "pz_decompress.hip"],
    "decode_kernel": ["pz_device.h", "pz_decompress.hip"],
    "decompress_kernel": ["pz_device.h", "pz_decompress.hip"],
}


def kernel_source_hash(kernel):
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel.split("<")[0]]:
        with open(os.path.join(ROOT, "lossless_bit_plane_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def batch_name(tensor_names):
    """Name of a batched launch over these tensors in the profile summaries."""
    return "batch(" + ",".join(tensor_names) + ")"


def measured_traffic(kernel, launch_names):
    """HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy)
    of the named launches of `kernel` (a tensor's name, or batch_name of a
    batched launch), summed, from the committed rocprofv3 summary; None when
    the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_gpt2xl_activations.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        prof = json.load(f)
    hashes = prof.get("source_hash")
    if not isinstance(hashes, dict) or hashes.get(kernel.split("<")[0]) != kernel_source_hash(kernel):
        return None, f"{kernel} changed since the counters in profiles/ were taken"
    total = 0.0
    for name in launch_names:
        t = prof["traffic"].get(f"{kernel}:{name}")
        if t is None:
            return None, f"no counters for {kernel} on {name}"
        total += t["fetch_bytes"] + t["write_bytes"]
    return round(total), "profiles/hbm_traffic_gpt2xl_activations.json (the batched launch)"


def host_threads():
    """Threads for the oracle: the job's CPU share where the host declares
    one (OMP_NUM_THREADS), else every core of this process's affinity mask;
    with the facts to report next to it."""
    affinity = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(share)) if share.isdigit() and int(share) > 0 else affinity
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, {"nproc": affinity, "os_cpu_count": os.cpu_count(), "cpu_model": model,
                     "omp_num_threads": share or None}


def cpu_baseline(tensors, sample_mb, gpu_streams):
    """The oracle, as it stands: chunk-parallel over the host threads on the
    whole workload (the reported value), and single-threaded on the same
    fraction of whole chunks from the start of every tensor (a bounded
    sample); compress then decompress, round trip checked. The oracle's
    streams of the whole workload are compared byte for byte with the GPU's
    (`gpu_streams`, by tensor name). Returns (baseline, equal by tensor)."""
    import oracle

    threads, host = host_threads()
    equal = {}

    def run(frac, nthreads):
        raw = 0
        t_c = t_d = 0.0
        for t in tensors:
            n = max(4096, int(t.nbytes * frac) // 4096 * 4096) if frac < 1.0 else t.nbytes
            part = t.data[:n]
            a = time.perf_counter()
            s = oracle.compress(part, t.elem_bits, threads=nthreads)
            b = time.perf_counter()
            back = oracle.decompress(s, n, t.elem_bits, threads=nthreads)
            c = time.perf_counter()
            assert np.array_equal(back, part)
            if frac >= 1.0:
                equal[t.name] = bool(np.array_equal(s, gpu_streams[t.name]))
            raw += n
            t_c += b - a
            t_d += c - b
        return raw, t_c, t_d

    total = sum(t.nbytes for t in tensors)
    raw, t_c, t_d = run(1.0, threads)
    log(f"cpu baseline: whole workload {raw / 1e6:.1f} MB, {threads} threads, "
        f"compress {t_c:.2f}s decompress {t_d:.2f}s; GPU streams equal to the oracle's: {equal}")
    frac1 = min(1.0, sample_mb * 1e6 / total)
    raw1, c1, d1 = run(frac1, 1)
    log(f"cpu baseline: {raw1 / 1e6:.1f} MB sample, 1 thread, compress {c1:.2f}s decompress {d1:.2f}s")
    return {
        "value": round(raw / (t_c + t_d) / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole workload ({raw / 1e6:.1f} MB), chunk-parallel on {threads} threads; "
                  f"compress {raw / t_c / 1e6:.1f} MB/s, decompress {raw / t_d / 1e6:.1f} MB/s",
        "host": host,
        "single_thread": {
            "value": round(raw1 / (c1 + d1) / 1e9, 5), "unit": "GB/s", "cores": 1,
            "sample": f"first {frac1 * 100:.1f}% (whole chunks) of each tensor, {raw1 / 1e6:.1f} MB; "
                      f"compress {raw1 / c1 / 1e6:.2f} MB/s, decompress {raw1 / d1 / 1e6:.2f} MB/s",
        },
    }, equal


def oracle_check(tensors, gpu_streams):
    """Byte-for-byte equality of the GPU streams with the oracle's streams of
    the same tensors (chunk-parallel oracle on the host threads), and the
    oracle's own compress and decompress rates on them (round trip checked).
    Returns (equal by tensor name, rates)."""
    import oracle

    threads, _ = host_threads()
    eq = {}
    raw = 0
    t_c = t_d = 0.0
    for t in tensors:
        a = time.perf_counter()
        s = oracle.compress(t.data, t.elem_bits, threads=threads)
        b = time.perf_counter()
        back = oracle.decompress(s, t.nbytes, t.elem_bits, threads=threads)
        c = time.perf_counter()
        assert np.array_equal(back, t.data)
        eq[t.name] = bool(np.array_equal(s, gpu_streams[t.name]))
        raw += t.nbytes
        t_c += b - a
        t_d += c - b
    log(f"oracle check: {eq}")
    return eq, {"threads": threads, "compress_raw_gbps": round(raw / t_c / 1e9, 4),
                "decompress_raw_gbps": round(raw / t_d / 1e9, 4)}


if __name__ == "__main__":
    main()
