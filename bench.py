"""Benchmark of the mask-aware attention forward path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
fmask_encode (compressed mask -> canonical intervals) -> fmask_classify
(exact tile table, compact lists, longest-first order) -> fmask_attn_fwd.
Inputs are resident in HBM before the timed region.

Headline workload: causal-document packing at 32768 tokens, batch 1, 32 query
heads, 8 K/V heads, head dim 128, bf16, document lengths drawn uniformly from
the multiples of 64 in [256, 4096].  value = effective TFLOP/s counting only
unmasked FLOPs: 4 * d * (visible (i, j) pairs) * heads / step time.

Also reported (one object each under "workloads"): the other workloads at
their full sizes, attention kernel time and effective TFLOP/s (gathered GB/s
for the selected-key workload).

Prints ONE JSON line.  --gpus N with N > 1 exits: the benchmark runs on one GPU.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_PROBE_BYTES = 256 << 20


def _bf16(torch, a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def visible_pairs(torch, enc):
    """Visible (i, j) pairs per mask, from the encoder's canonical intervals."""
    iv = enc.intervals().to(torch.int64)
    sq = enc.struct.sq
    masked = (iv[:, :, 1] - iv[:, :, 0]) + (iv[:, :, 3] - iv[:, :, 2])
    return (sq - masked).sum(dim=-1)  # [batch][heads]


def visible_pairs_bitmap(torch, enc):
    st, ix, bits, cnt = enc.bitmap()
    e = enc.struct
    n_full = 0
    st64 = st.to(torch.int64)
    # valid elements of every FULL block
    rows = torch.clamp(e.sq - torch.arange(e.nbq, device=st.device) * 64, max=64)
    cols = torch.clamp(e.skv - torch.arange(e.nbk, device=st.device) * 64, max=64)
    area = rows[:, None] * cols[None, :]
    n_full = ((st64 == 2) * area).sum(dim=(-1, -2))
    # popcount of the partial pool words, attributed to their mask
    words = bits.view(torch.int64)
    pc = torch.zeros_like(words)
    x = words.clone()
    for _ in range(64):
        pc += x & 1
        x = torch.bitwise_right_shift(x, 1) & 0x7FFFFFFFFFFFFFFF
    per_entry = pc.sum(dim=1)
    owner = torch.zeros(cnt, dtype=torch.int64, device=st.device)
    flat_ix = ix.reshape(e.batch * e.heads, -1)
    for m in range(e.batch * e.heads):
        sel = flat_ix[m][flat_ix[m] >= 0].to(torch.int64)
        owner[sel] = m
    part = torch.zeros(e.batch * e.heads, dtype=torch.int64, device=st.device)
    part.index_add_(0, owner, per_entry)
    return n_full + part.reshape(e.batch, e.heads)


EV_EVERY = 4  # timed steps per sampled attention launch (each recorded event costs the stream microseconds)
DATASHEET_SCLK_MHZ = 2400.0  # the clock PEAK_BF16_TFLOPS assumes


class ClockMonitor:
    """The GPU's graphics clock in MHz, sampled every ~2 ms from sysfs
    (pp_dpm_sclk: the level marked current) in a daemon thread between start()
    and stop().  Under sustained MFMA load the clock settles well below the
    datasheet's 2.4 GHz, so the bench also reports the fraction of the peak at
    the clock measured over the timed steps.  Inactive where the file is absent."""

    def __init__(self):
        import glob
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.samples = []
        self._stop = False
        self._thread = None

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):  # e.g. "1: 1749Mhz *"
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
        return None

    def _run(self):
        while not self._stop:
            try:
                v = self._read()
            except (OSError, ValueError, IndexError):
                v = None
            if v:
                self.samples.append(v)
            time.sleep(0.002)

    def start(self):
        if self.path:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop = True
        if self._thread:
            self._thread.join()
        if not self.samples:
            return None
        a = np.array(self.samples)
        return dict(mean=float(a.mean()), min=float(a.min()), max=float(a.max()), samples=int(a.size),
                    source=self.path)


def time_workload(torch, fm, synth, name, steps, warmup, min_warmup_s=0.5, graph=False, bm=None, blocks=False,
                  clock=False):
    w = synth.workload(name)
    q, k, v = (_bf16(torch, a) if w["dtype"] == "bf16" else torch.from_numpy(a).cuda()
               for a in synth.draw_qkv(w))
    mi = fm.MaskInput(w["mask"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    selected = w["mask"]["family"] == "selected_key"

    # the encoding and the tile table live in buffers the caller allocates once
    # (the library never allocates); every step re-runs the encoder and classifier
    enc0 = fm.encode(mi)
    # (bm: tile rows of the table; None = the library's preferred tile)
    tile = dict(bm=bm, bn=64) if bm else {}
    bufs = [enc0.buf, None if selected else fm.classify(enc0, dtype=w["dtype"], d=w["D"], **tile).buf]
    # (blocks: selected-key lists run in the block-major form, its workspace
    # allocated once like the other buffers)
    ws = (torch.empty(fm.attn_blocks_workspace_bytes(q, k, v, enc0), dtype=torch.uint8, device="cuda")
          if blocks else None)

    def step(ev=None, attn_only=False):
        # (each recorded event costs the stream a few microseconds, so the timed
        # steps record only the two around the attention launch, and that on
        # every EV_EVERY-th step; the encoder and classifier times come from a
        # separate pass that records all four)
        if ev and not attn_only:
            ev[0].record(stream)
        enc = fm.encode(mi, out=bufs[0])
        if ev and not attn_only:
            ev[1].record(stream)
        tiles = None if selected else fm.classify(enc, dtype=w["dtype"], d=w["D"], out=bufs[1], **tile)
        if ev:
            ev[2].record(stream)
        if blocks:
            fm.attn_fwd_blocks(q, k, v, enc, scale=w["scale"], out=o, lse=lse, workspace=ws)
        else:
            fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"], out=o, lse=lse)
        if ev:
            ev[3].record(stream)
        return enc, tiles

    # warm-up: at least `warmup` steps and half a second, so clocks have settled
    t_w = time.perf_counter()
    n_w = 0
    while n_w < warmup or time.perf_counter() - t_w < min_warmup_s:
        enc, tiles = step()
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    mon = ClockMonitor() if clock else None
    if mon:
        mon.start()
    t0 = time.perf_counter()
    for i in range(steps):
        # (events around every EV_EVERY-th attention launch of the timed region)
        enc, tiles = step(evs[i] if i % EV_EVERY == 0 else None, attn_only=True)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    sclk = mon.stop() if mon else None
    eager_wall = wall
    att = [a[2].elapsed_time(a[3]) for i, a in enumerate(evs) if i % EV_EVERY == 0]
    # breakdown pass (not timed): encoder and classifier launches
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evb[i])
    torch.cuda.synchronize()
    t_enc = np.mean([a[0].elapsed_time(a[1]) for a in evb])
    t_cls = np.mean([a[1].elapsed_time(a[2]) for a in evb])
    if graph:
        # The same step captured once as a HIP graph and replayed: every replay
        # runs the encoder, classifier and attention kernels again; only the
        # host's launch work between them is gone.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(max(warmup, 3)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
    t_att = np.mean(att)

    rec = dict(workload=name, B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], Sq=w["Sq"], Skv=w["Skv"], D=w["D"],
               dtype=w["dtype"], ms_per_step=wall * 1e3, encode_ms=float(t_enc),
               classify_ms=float(t_cls), attn_ms=float(t_att), eager_ms_per_step=eager_wall * 1e3,
               step_launch="hip graph replay" if graph else "eager",
               attn_ms_median=float(np.median(att)), attn_ms_min=float(np.min(att)))
    if sclk:
        rec["sclk_mhz"] = sclk
    if selected:
        rec["form"] = "block-major" if blocks else "per-query"
        ls, cn = enc.lists()
        cells = int(cn.sum().item()) * w["mask"]["sel_cells"]  # listed cells per (b, query)
        nvis = cells * w["Hq"]                                 # every head of the query
        gathered = cells * w["Hkv"] * 2 * w["D"] * 2            # K and V rows per kv head, bf16
        rec.update(visible_pairs=int(nvis), effective_tflops=4 * w["D"] * nvis / (t_att * 1e-3) / 1e12,
                   gathered_gbs=gathered / (t_att * 1e-3) / 1e9, gathered_bytes=int(gathered))
    else:
        if enc.kind == fm.ENC_INTERVALS:
            pairs = visible_pairs(torch, enc)
        else:
            pairs = visible_pairs_bitmap(torch, enc)
        mb, mh = enc.struct.batch, enc.struct.heads
        nvis = int(pairs.sum().item()) * (w["B"] // mb) * (w["Hq"] // mh)
        flops = 4 * w["D"] * nvis
        st = tiles.arrays()[0]
        rec.update(visible_pairs=int(nvis), effective_flop=int(flops),
                   effective_tflops=flops / (wall) / 1e12,
                   attn_effective_tflops=flops / (t_att * 1e-3) / 1e12,
                   tiles=dict(bm=tiles.struct.bm, bn=tiles.struct.bn,
                              skip=int((st == 0).sum().item()), partial=int((st == 1).sum().item()),
                              full=int((st == 2).sum().item())))
        if enc.kind == fm.ENC_INTERVALS:
            # the mask as the kernels read it (four int32 per key column and mask
            # slice) against a dense bool mask of the same slices
            rec["mask_bytes"] = dict(intervals=int(enc.intervals().numel() * 4),
                                     dense_bool=int(enc.struct.batch * enc.struct.heads * w["Sq"] * w["Skv"]))
        if "doc_lengths" in w:
            exp = sum(L * (L + 1) // 2 for L in w["doc_lengths"]) * w["B"] * w["Hq"]
            assert exp == nvis, (exp, nvis)
            rec["doc_lengths"] = w["doc_lengths"]
    del q, k, v, o, lse
    return rec


def time_decode(torch, fm, synth, name, steps, warmup):
    """Few-query selected-key attention: the one-pass kernel (one workgroup per
    query and K/V head) against the split form (lists split over workgroups,
    partial states merged), launch latency and gathered K/V bytes per second."""
    w = synth.workload(name)
    q, k, v = (_bf16(torch, a) for a in synth.draw_qkv(w))
    enc = fm.encode(w["mask"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, 64 << 20), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(max(warmup, 5)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    t1 = timed(lambda: fm.attn_fwd(q, k, v, enc, None, scale=w["scale"], out=o, lse=lse))
    ts = timed(lambda: fm.attn_fwd_split(q, k, v, enc, splits=0, scale=w["scale"], out=o, lse=lse,
                                         workspace=ws))
    ls, cn = enc.lists()
    cells = int(cn.sum().item()) * w["mask"]["sel_cells"]
    gathered = cells * w["Hkv"] * 2 * w["D"] * 2
    del q, k, v, o, lse, ws
    return dict(workload=name, B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], Sq=w["Sq"], Skv=w["Skv"], D=w["D"],
                dtype="bf16", one_pass_us=t1 * 1e3, split_us=ts * 1e3, gathered_bytes=int(gathered),
                split_gathered_gbs=gathered / (ts * 1e-3) / 1e9,
                one_pass_gathered_gbs=gathered / (t1 * 1e-3) / 1e9)


def time_dense_encode(torch, fm, synth, name, steps):
    """Dense-mask input: the workload's mask materialised as uint8 [Sq][Skv] on the
    device (from its compressed encoding), then encoded back from the dense form
    (automatic form; one synchronising flag read).  Reports the encode time and
    the dense vs compressed bytes."""
    w = synth.workload(name)
    S, K = w["Sq"], w["Skv"]
    # the dense input: the family's own encoding expanded on the device
    iv = fm.encode(w["mask"]).intervals()[0, 0].long()  # [4][K]
    dense = torch.empty((1, 1, S, K), dtype=torch.uint8, device="cuda")
    for r0 in range(0, S, 2048):
        rows = torch.arange(r0, min(S, r0 + 2048), device="cuda")[:, None]
        masked = ((iv[0] <= rows) & (rows < iv[1])) | ((iv[2] <= rows) & (rows < iv[3]))
        dense[0, 0, r0:r0 + rows.shape[0]] = (~masked).to(torch.uint8)
    spec = dict(family="dense", sq=S, skv=K, batch=1, heads=1, dense=dense)
    mi = fm.MaskInput(spec)
    enc = fm.encode(mi)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        enc = fm.encode(mi)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    comp = 4 * 4 * K if enc.kind == fm.ENC_INTERVALS else int(enc.buf.numel())
    del dense
    return dict(workload=name + "_dense_input", Sq=S, Skv=K, kind="intervals" if enc.kind == fm.ENC_INTERVALS
                else "bitmap", encode_ms=t * 1e3, dense_bytes=S * K, compressed_bytes=comp,
                dense_read_gbs=S * K / t / 1e9)


def time_backward(torch, fm, synth, name, steps, warmup):
    """Backward pass (fmask_attn_bwd) of a workload: attention-gradient launch time
    and effective TFLOP/s over 10 D flops per visible pair (QK^T, dO V^T, P^T dO,
    dS K, dS^T Q; the recomputation both gradient kernels do is not counted)."""
    w = synth.workload(name)
    q, k, v = (_bf16(torch, a) for a in synth.draw_qkv(w))
    do = _bf16(torch, synth.draw_dout(w))
    enc = fm.encode(w["mask"])
    tiles = fm.classify(enc, 128, 64)
    o, lse = fm.attn_fwd(q, k, v, enc, tiles, scale=w["scale"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fm.attn_bwd_workspace_bytes(q, k, v, o, tiles), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: fm.attn_bwd(q, k, v, o, lse, do, enc, tiles, scale=w["scale"], dq=dq, dk=dk, dv=dv,
                              workspace=ws)
    for _ in range(max(warmup, 3)):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps
    nvis = int(visible_pairs(torch, enc).sum().item()) * w["B"] * w["Hq"]
    flops = 10 * w["D"] * nvis
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return dict(workload=name + "_backward", B=w["B"], Hq=w["Hq"], Hkv=w["Hkv"], Sq=w["Sq"], Skv=w["Skv"],
                D=w["D"], dtype="bf16", bwd_ms=t, visible_pairs=nvis, effective_flop=flops,
                effective_tflops=flops / (t * 1e-3) / 1e12)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_causal_doc_32k_hbm_bytes.txt")
ATTN_SOURCES = [os.path.join(ROOT, "mask_aware_block_amd", "csrc", f)
                for f in ("attn_bf16_o3.hip", "attn_common.h", "device_util.h")]


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, or None if the kernel source changed since the counters were taken."""
    import hashlib
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        h = hashlib.sha256()
        for path in ATTN_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
        if fields.get("kernel_source_sha256") != sha:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(synth, name, rows, heads):
    """The float64 oracle on a bounded sample of the workload, same FLOP numerator."""
    from oracle import attention as OA
    from oracle import masks as OM
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w = synth.workload(name)
    q, k, v = synth.draw_qkv(w)
    q = OA.bf16_bits_to_f64(q[:, :heads, :rows])
    k = OA.bf16_bits_to_f64(k[:, :1])
    v = OA.bf16_bits_to_f64(v[:, :1])
    G = w["Hq"] // w["Hkv"]
    heads = min(heads, G)
    spec = w["mask"]
    vf = OA.spec_vis_fn(spec)
    t0 = time.perf_counter()
    OA.attention_dense(q[:, :heads], k, v, vf, w["scale"])
    dt = time.perf_counter() - t0
    nvis = int(np.asarray(OM.dense_vis(spec, 0, 0, np.arange(rows))).sum()) * heads
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        pass
    return dict(value=4 * w["D"] * nvis / dt / 1e12, unit="effective TFLOP/s", cores=int(threads),
                kind="oracle", seconds=dt, affinity=len(os.sched_getaffinity(0)), cpu_model=cpu,
                sample=f"{name}: query heads 0..{heads - 1} (K/V head 0), rows 0..{rows - 1} of {w['Sq']}, "
                       f"all {w['Skv']} keys, float64 dense masked softmax attention")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the 32K causal-document step (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as one captured HIP graph instead of launching its calls eagerly")
    ap.add_argument("--cpu-rows", type=int, default=32768)
    ap.add_argument("--cpu-heads", type=int, default=3,
                    help="query heads of the CPU-baseline sample (about 5 s of oracle work each)")
    ap.add_argument("--min-warmup-s", type=float, default=0.5,
                    help="warm up for at least this long (clocks settle); 0 for counter runs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward pass of the 32K causal-document workload "
                         "(for profiling runs); prints its own JSON line")
    ap.add_argument("--only", default=None,
                    help="time only this workload (a forward workload name, e.g. selected_key_128k) and print its "
                         "own JSON line (for profiling runs)")
    ap.add_argument("--blocks", action="store_true",
                    help="with --only on a selected-key workload: the block-major form")
    ap.add_argument("--bm", type=int, default=None,
                    help="with --only: tile rows of the table (default: the library's preferred tile)")
    ap.add_argument("--dense-only", action="store_true",
                    help="time only the dense-mask encode of the 8K causal-document mask (for profiling runs); "
                         "prints its own JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import mask_aware_block_amd as fm
    import synth

    fm.lib()
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.backward_only:
        print(json.dumps(time_backward(torch, fm, synth, "causal_doc_32k", args.steps, args.warmup)))
        return
    if args.dense_only:
        print(json.dumps(time_dense_encode(torch, fm, synth, "causal_doc_8k", args.steps)))
        return
    if args.only:
        print(json.dumps(time_workload(torch, fm, synth, args.only, args.steps, args.warmup, args.min_warmup_s,
                                       bm=args.bm, blocks=args.blocks)))
        return
    # (--graph: steps of mask families whose encoder records kernel launches
    # only are replayed as one HIP graph; on this stack that measured slower
    # than launching them eagerly, so eager is the default.)
    graphable = {"causal_doc_32k", "causal_doc_8k", "shared_question_32k", "band_32k", "band_neg_4k"}
    head = time_workload(torch, fm, synth, "causal_doc_32k", args.steps, args.warmup, args.min_warmup_s,
                         graph=args.graph, clock=True)
    others = []
    if not args.headline_only:
        for name in ("causal_doc_8k", "shared_question_32k", "band_32k", "band_neg_4k", "varlen_prefill_32k",
                     "block_bitmap_16k", "tree_4k", "selected_key_128k"):
            others.append(time_workload(torch, fm, synth, name, max(3, args.steps // 2), 2,
                                        min(0.2, args.min_warmup_s), graph=name in graphable and args.graph))
            torch.cuda.empty_cache()
        # the sparse block mask again on the 64 x 64 table (two block rows per
        # workgroup, each walking its own list), and the selected-key lists in
        # the block-major form
        others.append(time_workload(torch, fm, synth, "block_bitmap_16k", max(3, args.steps // 2), 2,
                                    min(0.2, args.min_warmup_s), bm=64))
        torch.cuda.empty_cache()
        others.append(time_workload(torch, fm, synth, "selected_key_128k", max(3, args.steps // 2), 2,
                                    min(0.2, args.min_warmup_s), blocks=True))
        torch.cuda.empty_cache()
        for name in ("causal_doc_8k", "causal_doc_32k"):
            others.append(time_backward(torch, fm, synth, name, max(3, args.steps // 4), 2))
            torch.cuda.empty_cache()
        for name in ("selected_key_decode_128k", "selected_key_decode16_128k"):
            others.append(time_decode(torch, fm, synth, name, max(20, args.steps), 5))
            torch.cuda.empty_cache()
        others.append(time_dense_encode(torch, fm, synth, "causal_doc_8k", 5))

    achieved = head["effective_flop"] / (head["attn_ms"] * 1e-3) / 1e12
    out = {
        "metric": "effective TFLOP/s (unmasked FLOPs) + fraction of bf16 MFMA peak, 8K-128K seq",
        "value": head["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, seeded document lengths)",
        "config": {"workload": "causal_document_32k", "step_launch": head["step_launch"],
                   "eager_ms_per_step": head["eager_ms_per_step"], "batch": 1, "q_heads": 32, "kv_heads": 8,
                   "seq_len": 32768, "head_dim": 128, "doc_lengths": head["doc_lengths"],
                   "visible_pairs": head["visible_pairs"], "mask_bytes": head.get("mask_bytes")},
        "fraction_of_peak": head["effective_tflops"] / PEAK_BF16_TFLOPS,
        "step_breakdown_ms": {"encode": head["encode_ms"], "classify": head["classify_ms"],
                              "attention": head["attn_ms"]},
        "roofline": {"bound": "mfma", "kernel": "k_attn_o3<128> (128x64 tiles, intervals)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic()},
        # the same peak scaled to the graphics clock measured over the timed steps
        # (null where the clock cannot be read)
        "sclk_mhz": head.get("sclk_mhz"),
        "workloads": others,
    }
    if head.get("sclk_mhz"):
        f = head["sclk_mhz"]["mean"] / DATASHEET_SCLK_MHZ
        out["roofline"]["peak_at_sclk"] = PEAK_BF16_TFLOPS * f
        out["roofline"]["frac_at_sclk"] = achieved / (PEAK_BF16_TFLOPS * f)
        out["fraction_of_peak_at_sclk"] = head["effective_tflops"] / (PEAK_BF16_TFLOPS * f)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(synth, "causal_doc_32k", args.cpu_rows, args.cpu_heads)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
