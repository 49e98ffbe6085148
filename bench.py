#!/usr/bin/env python
"""Throughput of the sparse masked MHA forward path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input
already resident in device memory:
    encode the [S, S] mask (GPU, 2 or 3 launches)  ->  attention forward in
    one launch that picks the row-wise or block-wise algorithm with the cost
    model evaluated on the device from the encoding's statistics.
No host synchronisation inside a step, so steps are captured into a HIP
graph and replayed (--eager launches every step from the host instead).
Kernel durations (encode_ms, fwd_ms, and the roofline's) come from HIP
events around graphs of back-to-back launches of that part alone.
The headline value is effective TFLOP/s: 4*d FLOPs per valid (query, key)
pair, summed over every (batch, head), divided by the step time.

Default workload (the headline): the long-sequence unstructured mask
(B=1, H=32, S=16384, d=128, bf16 in, fp32 out, causal AND (|i-j| <= 1024
OR Bernoulli(0.02))).  With the default options the line also carries
`per_mask`: the same measurements on each of the five workloads (warm: the
inputs stay in the caches between launches; cold: launches rotate through
copies of the inputs, more than 1 GiB in all where memory allows, twice
the 256 MB last-level cache).  --seq-len changes S (any length: the last
tiles are cut), --mask-stack batch gives each sequence its own mask (the
pattern cut to a per-sequence length), encoded as one stack.  Prints one
JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}   # dense, MI355X
HBM_PEAK_GBS = 8000.0
RIDGE = MFMA_PEAK_TFLOPS["f16"] * 1e12 / (HBM_PEAK_GBS * 1e9)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id 1..7 (default 5, the 16k mask; 6 = "
                         "the row-wise kernel's regime, a 0.1%% random "
                         "mask; 7 = workload 5's far tiles alone)")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "rowwise", "blockwise",
                             "blockwise_dense"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle baseline (0 disables)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from the host instead of "
                         "replaying a captured HIP graph")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy "
                         "(the reference for scaling FETCH_SIZE/WRITE_SIZE "
                         "counter readings to bytes)")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="FETCH_SIZE and WRITE_SIZE counter CSVs of this "
                         "bench (rocprofv3 --pmc, one counter per run), then "
                         "those of --copy-reference; writes the HBM bytes "
                         "per launch of the attention kernel to profiles/")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="override the workload's S (mask pattern and Q/K/V "
                         "regenerated at that length)")
    ap.add_argument("--mask-stack", default="shared",
                    choices=["shared", "batch"],
                    help="shared: one mask for every (batch, head); batch: "
                         "one mask per sequence (padding to a seeded length "
                         "in [S/2, S])")
    ap.add_argument("--mask-source", default="dense",
                    choices=["dense", "pattern"],
                    help="dense: encode the stored [S, S] mask; pattern: "
                         "encode from the workload's pattern (no dense mask "
                         "on the device; BigBird and long_random then draw "
                         "their random elements from the pattern's "
                         "generator)")
    ap.add_argument("--epilogue", default="none", choices=["none", "out_proj"],
                    help="out_proj: the step also runs the fused output "
                         "projection (attention output x W^T + bias + "
                         "residual, D = H*d) on the attention output")
    ap.add_argument("--per-mask", default="auto",
                    choices=["auto", "on", "off"],
                    help="also measure workloads 1-5 (per_mask); auto = on "
                         "for the default headline options")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache timings (rotated input "
                         "copies)")
    ap.add_argument("--out-dtype", default="auto",
                    choices=["auto", "in", "f32"],
                    help="output type; auto = input type for fp16, f32 for "
                         "bf16")
    return ap.parse_args()


COPY_REF_BYTES = 256 << 20
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def copy_reference():
    """A plain copy of COPY_REF_BYTES, five times (one kernel each)."""
    import torch
    x = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes": COPY_REF_BYTES}))


def source_digest():
    """Digest of the HIP sources: counter readings are valid only for the
    kernels they were taken on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_masked_head_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from committed counter
    readings (profiles/traffic_<kernel>_<workload>.json), or None when they
    were taken on other sources."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_digest") != source_digest():
        return None
    return rec["hbm_bytes_per_launch"]


def _counter_kib(path, name_part):
    """Mean per-dispatch value of the one counter in a rocprofv3 counter CSV
    over the dispatches of kernels whose name contains name_part."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if name_part in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + \
                float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatch of *{name_part}* in {path}")
    return sum(per.values()) / len(per), len(per)


def write_traffic(args, cfg):
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.write_traffic
    kern = "auto_fwd" if args.kernel == "auto" else f"{args.kernel}_fwd"
    f_kib, nf = _counter_kib(fetch_csv, kern)
    w_kib, nw = _counter_kib(write_csv, kern)
    # torch runs a same-type contiguous copy as the runtime's copyBuffer
    # kernel; the fill that creates the source is a different kernel
    cf_kib, _ = _counter_kib(cfetch_csv, "copyBuffer")
    cw_kib, _ = _counter_kib(cwrite_csv, "copyBuffer")
    # counter KiB that one true byte reads as, for a plain copy
    ff = cf_kib * 1024.0 / COPY_REF_BYTES
    fw = cw_kib * 1024.0 / COPY_REF_BYTES
    rec = {"kernel": kern, "workload": cfg.name,
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
           "dispatches": [nf, nw],
           "copy_reference_bytes": COPY_REF_BYTES,
           "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
           "fetch_scale": ff, "write_scale": fw,
           "hbm_read_bytes_per_launch": f_kib * 1024.0 / ff,
           "hbm_write_bytes_per_launch": w_kib * 1024.0 / fw,
           "hbm_bytes_per_launch": f_kib * 1024.0 / ff + w_kib * 1024.0 / fw,
           "source_digest": source_digest()}
    os.makedirs(TRAFFIC_DIR, exist_ok=True)
    out = os.path.join(TRAFFIC_DIR, f"traffic_{kern}_{cfg.name}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def encoding_bytes(st, rows):
    return 4 * 2 * (rows + 1) + 4 * (st["n_full"] + st["n_partial"]) + \
        512 * st["n_partial"]


def users_per_mask(mask, B, H):
    """(batch, head) pairs that share each mask of a [S, S] mask or a
    [mask_b, mask_h, S, S] stack."""
    if mask.ndim == 2:
        return B * H
    return (1 if mask.shape[0] > 1 else B) * (1 if mask.shape[1] > 1 else H)


def cpu_baseline(cfg, mask, qkv, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload.

    The dense fp64 oracle costs the same for every query row, so the time
    of the whole workload is the encoder's time plus the attention time of
    the sampled rows scaled by (all rows / sampled rows)."""
    import numpy as np
    from oracle.attention import attention_rows
    from oracle.encode import encode_c
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    from oracle.encode import encode_stack
    t0 = time.perf_counter()
    encode_c(mask) if mask.ndim == 2 else encode_stack(mask)
    t_enc = time.perf_counter() - t0
    rows_done = 0
    t_attn = 0.0
    blk = min(cfg.S, 1024)
    q, k, v = qkv
    for b in range(cfg.B):
        for h in range(cfg.H):
            for r0 in range(0, cfg.S, blk):
                r1 = min(cfg.S, r0 + blk)
                t1 = time.perf_counter()
                attention_rows(q, k, v, mask, b, h, np.arange(r0, r1))
                t_attn += time.perf_counter() - t1
                rows_done += r1 - r0
                if t_attn >= budget_s:
                    break
            if t_attn >= budget_s:
                break
        if t_attn >= budget_s:
            break
    total_rows = cfg.B * cfg.H * cfg.S
    t_total = t_enc + t_attn * total_rows / rows_done
    flops = 4.0 * cfg.d * users_per_mask(mask, cfg.B, cfg.H) * float(mask.sum())
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s",
            "cores": int(cores), "kind": "oracle",
            "sample": (f"scalar C encoder on the full mask + fp64 dense "
                       f"attention oracle on {rows_done} of {total_rows} "
                       f"query rows ({rows_done // cfg.S} heads), "
                       f"extrapolated per row; {t_total:.2f} s estimated "
                       f"for the whole workload")}


def workload(args):
    """The Config and mask ([S, S], or a [B, 1, S, S] stack) the options
    name."""
    import dataclasses
    from workloads import get_config, make_mask, padding_stack
    cfg = get_config(args.config)
    if args.seq_len:
        cfg = dataclasses.replace(
            cfg, S=args.seq_len, name=f"{cfg.name}-S{args.seq_len}",
            desc=f"{cfg.desc}; S changed to {args.seq_len}")
    if args.mask_source == "pattern":
        from oracle.pattern import pattern_mask   # the mask, for FLOPs and the CPU leg
        from workloads import pattern_of
        if args.mask_stack != "shared":
            raise SystemExit("--mask-source pattern takes one shared mask")
        pat = pattern_of(cfg)
        mask = pattern_mask(cfg.S, **pat)
        cfg = dataclasses.replace(
            cfg, name=f"{cfg.name}-pattern",
            desc=f"{cfg.desc}; encoded from its pattern")
        return cfg, mask
    mask = make_mask(cfg)
    if args.mask_stack == "batch":
        mask = padding_stack(mask, cfg.B, cfg.cid)
        cfg = dataclasses.replace(
            cfg, name=f"{cfg.name}-per-sequence",
            desc=f"{cfg.desc}; one mask per sequence (cut to a seeded length "
                 f"in [S/2, S])")
    return cfg, mask


COLD_BYTES = 1 << 30     # rotation target: twice the 256 MB last-level cache, x2
COLD_MAX_COPIES = 1024


def roofline_of(flops, nbytes, t_s, dtype):
    """Roofline entry of a kernel doing `flops` effective FLOPs and moving
    `nbytes` algorithmic bytes in `t_s` seconds: the bound is the one its
    arithmetic intensity puts it under."""
    if flops / nbytes < RIDGE:
        r = {"bound": "hbm", "achieved": nbytes / t_s / 1e9,
             "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": flops / t_s / 1e12,
             "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["algorithmic_flops"] = flops
    r["algorithmic_bytes"] = nbytes
    return r


class Timer:
    """Average duration of one call of a function's kernels: `reps` calls
    back to back captured in one graph (or launched eagerly), bracketed by
    events on their stream."""

    def __init__(self, stream, eager):
        self.stream, self.eager = stream, eager

    def us(self, fn, reps=20):
        import torch
        calls = fn if isinstance(fn, list) else [fn]
        if len(calls) > 1:
            reps = max(reps, len(calls))
        seq = [calls[i % len(calls)] for i in range(reps)]
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        if self.eager:
            for f in calls:
                f()
            torch.cuda.synchronize()
            a.record(self.stream)
            for f in seq:
                f()
            b.record(self.stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / reps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in seq:
                f()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):          # the median of three replays
            a.record(self.stream)
            g.replay()
            b.record(self.stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3 / reps)
        return sorted(ts)[1]


class Workload:
    """Device tensors of one workload and the calls a step makes."""

    def __init__(self, args, cfg, mask, dev, copies=1):
        import torch
        import sparse_masked_head_amd as smh
        from workloads import make_qkv
        self.cfg, self.mask, self.args = cfg, mask, args
        self.smh = smh
        qkv = make_qkv(cfg.B, cfg.H, cfg.S, cfg.d, cfg.dtype, seed=cfg.cid)
        self.qkv_host = qkv
        q, k, v = (x.to(dev) for x in qkv)
        self.in_dtype = q.dtype
        self.out_dt = {"auto": torch.float32 if cfg.dtype == "bf16"
                       else q.dtype, "in": q.dtype,
                       "f32": torch.float32}[args.out_dtype]
        self.mb, self.mh = (1, 1) if mask.ndim == 2 else mask.shape[:2]
        self.pattern = None
        mask_d = None
        if args.mask_source == "pattern":
            from workloads import pattern_of
            pat = dict(pattern_of(cfg))
            if pat.get("blocks") is not None:
                pat["blocks"] = torch.from_numpy(pat["blocks"]).to(dev)
            self.pattern = pat
        else:
            mask_d = torch.from_numpy(mask).to(dev)
        ws_bytes = smh.encode_workspace_bytes(cfg.S, self.mb, self.mh)
        self.sets = []
        for c in range(copies):
            qc, kc, vc = (q, k, v) if c == 0 else (x.clone() for x in (q, k, v))
            mc = mask_d if (c == 0 or mask_d is None) else mask_d.clone()
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            out = torch.empty(q.shape, dtype=self.out_dt, device=dev)
            self.sets.append({"q": qc, "k": kc, "v": vc, "mask": mc,
                              "ws": ws, "out": out})
        self.dev = dev
        for c in range(copies):
            self.sets[c]["enc"] = self.encode(c)
        torch.cuda.synchronize()
        self.stats = smh.mask_stats_get(self.sets[0]["enc"])
        self.kernel = args.kernel if args.kernel != "auto" else \
            smh.select_kernel(self.stats, cfg.B, cfg.H, cfg.d, q.dtype)
        per = sum(t.numel() * t.element_size() for t in
                  (self.sets[0][x] for x in ("q", "k", "v", "out", "ws")))
        if mask_d is not None:
            per += mask_d.numel() * mask_d.element_size()
        self.copy_bytes = per

    def encode(self, c=0):
        st = self.sets[c]
        if self.pattern is not None:
            return self.smh.encode_pattern(self.cfg.S, device=self.dev,
                                           workspace=st["ws"], **self.pattern)
        return self.smh.encode_mask(st["mask"], workspace=st["ws"])

    def fwd(self, c=0):
        st = self.sets[c]
        self.smh.sparse_mha_fwd(st["q"], st["k"], st["v"], st["enc"],
                                kernel=self.args.kernel,
                                out_dtype=self.out_dt, out=st["out"])

    def step(self, c=0):
        st = self.sets[c]
        st["enc"] = self.encode(c)
        self.fwd(c)

    # algorithmic work of one step
    def work(self):
        cfg, st = self.cfg, self.stats
        users = users_per_mask(self.mask, cfg.B, cfg.H)
        flops = 4.0 * cfg.d * users * st["nnz"]
        tiles = st["n_full"] + st["n_partial"]
        tile_flops = 4.0 * cfg.d * 4096.0 * users * tiles
        rows = self.mb * self.mh * cfg.n_ot
        enc_b = encoding_bytes(st, rows)
        eb_out = self.sets[0]["out"].element_size()
        attn_bytes = cfg.B * cfg.H * cfg.S * cfg.d * (3 * 2 + eb_out) + enc_b
        mask_bytes = 0 if self.pattern is not None else self.mask.size
        return flops, tile_flops, attn_bytes, mask_bytes + enc_b


def measure(args, cfg, mask, dev, timer, cold):
    """Warm (and cold) kernel timings of one workload: a dict for
    per_mask, and the Workload (for the headline's own timed steps)."""
    import torch
    w = Workload(args, cfg, mask, dev)
    flops, tile_flops, attn_bytes, enc_bytes = w.work()
    enc_us = timer.us(lambda: w.encode(0))
    fwd_us = timer.us(lambda: w.fwd(0))
    step_us = timer.us(lambda: w.step(0))
    dt = cfg.dtype
    e = {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "S": cfg.S, "d": cfg.d,
         "dtype": dt, "out_dtype": str(w.out_dt).replace("torch.", ""),
         "mask": cfg.desc, "kernel": w.kernel, "mask_stats": w.stats,
         "encode_ms": enc_us / 1e3, "fwd_ms": fwd_us / 1e3,
         "step_ms": step_us / 1e3,
         "fwd_tflops": flops / fwd_us / 1e6,
         "fwd_pct_mfma_peak": 100.0 * flops / fwd_us / 1e6 /
         MFMA_PEAK_TFLOPS[dt],
         "step_tflops": flops / step_us / 1e6,
         "tile_mfma_frac": tile_flops / fwd_us / 1e6 / MFMA_PEAK_TFLOPS[dt],
         "roofline": roofline_of(flops, attn_bytes, fwd_us * 1e-6, dt),
         "encoder": {"us": enc_us, "algorithmic_bytes": enc_bytes,
                     "achieved": enc_bytes / enc_us / 1e3, "unit": "GB/s",
                     "peak": HBM_PEAK_GBS,
                     "frac": enc_bytes / enc_us / 1e3 / HBM_PEAK_GBS}}
    e["roofline"]["kernel"] = "auto_fwd" if args.kernel == "auto" \
        else f"{w.kernel}_fwd"
    pred_row, pred_blk = w.smh.select_costs(w.stats, cfg.B, cfg.H, cfg.d,
                                            w.in_dtype)
    e["selector_pred_us"] = {"rowwise": pred_row, "blockwise": pred_blk}
    if cold:
        n = max(2, min(COLD_MAX_COPIES, -(-COLD_BYTES // w.copy_bytes)))
        del w
        torch.cuda.empty_cache()
        wc = Workload(args, cfg, mask, dev, copies=n)
        ce = timer.us([lambda c=c: wc.encode(c) for c in range(n)])
        cf = timer.us([lambda c=c: wc.fwd(c) for c in range(n)])
        cs = timer.us([lambda c=c: wc.step(c) for c in range(n)])
        e["cold"] = {"encode_ms": ce / 1e3, "fwd_ms": cf / 1e3,
                     "step_ms": cs / 1e3, "copies": n,
                     "rotation_bytes": n * wc.copy_bytes,
                     "fwd_tflops": flops / cf / 1e6,
                     "roofline": roofline_of(flops, attn_bytes, cf * 1e-6, dt)}
        del wc
        torch.cuda.empty_cache()
    return e


def main():
    args = parse()
    if args.copy_reference:
        copy_reference()
        return
    if args.write_traffic:
        write_traffic(args, workload(args)[0])
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus "
              f"{args.gpus} is not supported (the path needs no collective; "
              f"run --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_masked_head_amd as smh
    from workloads import get_config, make_mask

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    timer = Timer(stream, args.eager)
    cfg, mask = workload(args)
    w = Workload(args, cfg, mask, dev)
    q = w.sets[0]["q"]
    st = w.stats

    proj = None
    if args.epilogue == "out_proj":
        if w.out_dt != q.dtype:
            raise SystemExit("--epilogue out_proj needs the attention output "
                             "in the input type (--out-dtype in)")
        D = cfg.H * cfg.d
        g = torch.Generator().manual_seed(cfg.cid + 77)
        pw = (torch.randn(D, D, generator=g) / D ** 0.5).to(q.dtype).to(dev)
        pb = (0.1 * torch.randn(D, generator=g)).to(q.dtype).to(dev)
        pr = torch.randn(cfg.B, cfg.S, D, generator=g).to(q.dtype).to(dev)
        pout = torch.empty_like(pr)
        proj = (pw, pb, pr, pout)

    def step():
        w.step(0)
        if proj is not None:
            smh.out_proj(w.sets[0]["out"], proj[0], proj[1], proj[2],
                         out=proj[3])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # A step enqueues its kernels and needs no host synchronisation, so it
    # is captured once into a HIP graph and replayed (launch-bound
    # otherwise at small sizes).  `per_graph` steps per replay.
    per_graph = 1 if args.eager else max(1, min(10, args.steps))
    if args.steps % per_graph:
        per_graph = 1
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                step()
        torch.cuda.synchronize()
        graph.replay()          # warm replay
        torch.cuda.synchronize()

    t0 = time.perf_counter()
    if graph is None:
        for _ in range(args.steps):
            step()
    else:
        for _ in range(args.steps // per_graph):
            graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    del graph

    enc_ms = timer.us(lambda: w.encode(0)) / 1e3
    fwd_ms = timer.us(lambda: w.fwd(0)) / 1e3
    epi = None
    if proj is not None:
        p_us = timer.us(lambda: smh.out_proj(w.sets[0]["out"], proj[0],
                                             proj[1], proj[2], out=proj[3]))
        M, K, D = cfg.B * cfg.S, cfg.H * cfg.d, proj[0].shape[0]
        p_flops = 2.0 * M * K * D
        p_bytes = 2.0 * (M * K + D * K + D + 2 * M * D)
        epi = {"kernel": "out_proj", "us": p_us, "M": M, "K": K, "N": int(D),
               "tflops": p_flops / p_us / 1e6,
               "roofline": roofline_of(p_flops, p_bytes, p_us * 1e-6,
                                       cfg.dtype)}

    flops, tile_flops, attn_bytes, enc_bytes = w.work()
    value = flops / step_s / 1e12
    fwd_s = fwd_ms / 1e3
    roof = roofline_of(flops, attn_bytes, fwd_s, cfg.dtype)
    roof["kernel"] = "auto_fwd" if args.kernel == "auto" else f"{w.kernel}_fwd"
    roof["traffic"] = stored_traffic(roof["kernel"], cfg.name)
    pred_row, pred_blk = smh.select_costs(st, cfg.B, cfg.H, cfg.d, q.dtype)
    encoder = {"us": enc_ms * 1e3, "algorithmic_bytes": enc_bytes,
               "achieved": enc_bytes / (enc_ms * 1e-3) / 1e9, "unit": "GB/s",
               "peak": HBM_PEAK_GBS}
    encoder["frac"] = encoder["achieved"] / HBM_PEAK_GBS
    qkv_host = w.qkv_host
    del w, proj
    torch.cuda.empty_cache()

    per_mask = None
    default_opts = (args.seq_len == 0 and args.mask_stack == "shared" and
                    args.mask_source == "dense" and args.kernel == "auto" and
                    args.epilogue == "none" and args.out_dtype == "auto")
    if args.per_mask == "on" or (args.per_mask == "auto" and default_opts and
                                 args.config == 5):
        per_mask = []
        for cid in (1, 2, 3, 4, 5):
            c = get_config(cid)
            m = mask if c.name == cfg.name and args.seq_len == 0 else \
                make_mask(c)
            per_mask.append(measure(args, c, m, dev, timer,
                                    not args.no_cold))
            print(f"bench.py: per_mask {c.name} done", file=sys.stderr,
                  flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, mask, qkv_host, args.cpu_seconds)

    line = {
        "metric": "effective TFLOP/s on valid QK pairs (4*d FLOPs per valid "
                  "(query,key) pair) + % of MI355X dense MFMA peak, per mask",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_s * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded mask)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "S": cfg.S,
                   "d": cfg.d, "mask": cfg.desc,
                   "mask_stack": [int(x) for x in (mask.shape[:2]
                                                   if mask.ndim == 4
                                                   else (1, 1))],
                   "out_dtype": w_out_dtype(args, cfg),
                   "launch": "eager" if args.eager else
                   f"hip graph, {per_graph} steps per replay",
                   "parallelism": "single GPU"},
        "pct_mfma_peak": 100.0 * value / MFMA_PEAK_TFLOPS[cfg.dtype],
        "kernel": smh.select_kernel(st, cfg.B, cfg.H, cfg.d, q.dtype)
        if args.kernel == "auto" else args.kernel,
        "encode_ms": enc_ms, "fwd_ms": fwd_ms,
        "fwd_tflops": flops / fwd_s / 1e12,
        "fwd_pct_mfma_peak": 100.0 * flops / fwd_s / 1e12 /
        MFMA_PEAK_TFLOPS[cfg.dtype],
        "tile_mfma_frac": tile_flops / fwd_s / 1e12 /
        MFMA_PEAK_TFLOPS[cfg.dtype],
        "selector_pred_us": {"rowwise": pred_row, "blockwise": pred_blk},
        "mask_stats": st,
        "roofline": roof,
        "encoder": encoder,
        "epilogue": epi,
        "per_mask": per_mask,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def w_out_dtype(args, cfg):
    if args.out_dtype == "f32" or (args.out_dtype == "auto" and
                                   cfg.dtype == "bf16"):
        return "float32"
    return "float16" if cfg.dtype == "f16" else "bfloat16"


if __name__ == "__main__":
    main()
