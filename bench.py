"""Benchmark of the blockwise ring-attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the forward (ring walk, masks, online softmax, P.V) followed by the backward
(Delta preprocess, dK/dV kernel, dQ kernel), all through the C-ABI.  The
default workload is one device's share of a 1M-token context: ring rank 7 of
8, 131072 local queries against 1048576 keys, 16 heads, head_dim 64, bf16,
causal, with fully masked blocks skipped.

Prints one JSON line.  value = whole-step attention TFLOP/s, counting 4*D
(forward) + 10*D (backward) FLOPs per visible (query, key) pair.  Per-kernel
durations come from HIP events recorded on the stream the kernels run on.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd, fwd+bwd) at 1 MI355X and % of bf16 MFMA peak"
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    """Hash of every kernel source file: HBM counter figures are valid only for this exact code."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_exact_attn_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cuh"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (calibrated FETCH_SIZE + WRITE_SIZE) recorded in
    profiles/traffic_<workload>.txt, or None when absent or taken on other kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec, cur = {}, None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("source:"):
                rec["source"] = line.split(":", 1)[1].strip()
            elif line.startswith("kernel:"):
                cur = line.split(":", 1)[1].strip()
            elif line.startswith("hbm_bytes:") and cur:
                rec[cur] = int(float(line.split(":", 1)[1]))
    if rec.get("source") != kernel_source_hash():
        return None
    return rec.get(kernel)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="share-1m-r7")
    ap.add_argument("--ring-rank", type=int, default=None,
                    help="for a one-rank workload: time ring rank r instead (a sweep line, not the bench line)")
    ap.add_argument("--fwd-only", action="store_true", help="time the forward alone (not the bench line)")
    ap.add_argument("--ring-steps", action="store_true",
                    help="with a one-rank workload: run the pass as the per-step path a multi-GPU ring calls "
                         "(one ra_blockwise_attn_fwd_step / _bwd_step per visible ring step, then the "
                         "finalize calls), K/V blocks already in contiguous receive buffers (a sweep line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ffn", action="store_true",
                    help="time the blockwise SwiGLU feed-forward instead (a sweep line): one device's 131072 tokens, "
                         "d_model 1024, d_ff 2816, chunks of --ffn-chunk tokens, forward + backward")
    ap.add_argument("--ffn-chunk", type=int, default=16384, help="tokens per chunk of the blockwise feed-forward")
    ap.add_argument("--cpu-rows", type=int, default=256,
                    help="query rows in the oracle's fixed seeded sample (cpu_baseline)")
    ap.add_argument("--source-hash", action="store_true", help="print the kernel source hash and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, run one plain device copy of this many MiB (a known-size kernel "
                         "that calibrates the profiler's HBM byte counters)")
    return ap.parse_args()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, t, n_rows):
    """The float64 oracle, as it stands, on a fixed seeded sample of the same workload: n_rows query rows
    of head 0 (the first rows of a permutation drawn with seed 5) plus the first and last row of every ring
    block the queries span, each against its full visible key set, forward + backward.  Returns TFLOP/s
    over the sample's visible pairs and the time the oracle would take for the whole workload at the
    sample's rate (pairs of every head and batch row)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    h = 0
    f64 = lambda x: x.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    k = f64(t["k"][:, :, h:h + 1])
    v = f64(t["v"][:, :, h:h + 1])
    bias = None if t["bias"] is None else f64(t["bias"][h:h + 1])
    seg = None if t["segment_ids"] is None else t["segment_ids"].cpu().numpy()
    qpos_all = w.q_positions()
    rows = set(np.random.default_rng(5).permutation(w.q_len)[:n_rows].tolist())
    for start in range(0, w.q_len, w.block_len):
        rows.update((start, min(w.q_len, start + w.block_len) - 1))
    rows = np.array(sorted(rows), dtype=np.int64)
    pairs, elapsed, batch = 0, 0.0, 8
    for i0 in range(0, len(rows), batch):
        r = rows[i0:i0 + batch]
        q = f64(t["q"][:, r][:, :, h:h + 1])
        g = f64(t["dout"][:, r][:, :, h:h + 1]) if t.get("dout") is not None else np.ones_like(q)
        t0 = time.perf_counter()
        oracle.forward(q, k, v, q_pos=qpos_all[r], causal=w.causal, bias=bias, segment_ids=seg)
        oracle.backward(q, k, v, g, q_pos=qpos_all[r], causal=w.causal, bias=bias, segment_ids=seg)
        elapsed += time.perf_counter() - t0
        pairs += int(oracle.visible_pairs(qpos_all[r], w.kv_len, w.causal, seg))
    all_pairs = int(oracle.visible_pairs(qpos_all, w.kv_len, w.causal, seg)) * w.heads * (1 if seg is not None
                                                                                          else w.batch)
    fl = 14 * w.head_dim * pairs
    return {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "full_workload_s_extrapolated": round(elapsed * all_pairs / max(pairs, 1), 1),
            "sample": f"{len(rows)} query rows of head 0 (the first {n_rows} of a permutation drawn with seed 5, "
                      f"plus the first and last row of each ring block), each against its full visible key set, "
                      f"float64 forward+backward; {pairs} visible pairs in {elapsed:.1f} s"}


def gpu_clocks():
    """The GPU's current clocks, read from the driver's sysfs clock tables (no child process): the mean
    over the graphics clock domains and the memory clock, in MHz, or None where they cannot be read."""
    import glob
    import re

    def current(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*mhz", line, re.I)
                        if m:
                            return float(m.group(1))
        except OSError:
            pass
        return None
    gfx, mem = [], []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        g = current(os.path.join(dev, "pp_dpm_sclk"))
        if g is None:
            continue
        gfx.append(g)
        m = current(os.path.join(dev, "pp_dpm_mclk"))
        if m is not None:
            mem.append(m)
    if not gfx:
        return None
    return {"gfx_mean": round(sum(gfx) / len(gfx), 1), "gfx_min": min(gfx), "gfx_max": max(gfx),
            "mem": mem[0] if mem else None}


class ClockSampler:
    """Reads the clocks just before the timed region, every second or so during it (a thread reading sysfs;
    the GPU work is not touched) and just after it."""

    def __init__(self):
        import threading
        self.samples, self.before, self.after = [], None, None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            c = gpu_clocks()
            if c:
                self.samples.append(c["gfx_mean"])
            self._stop.wait(0.5)

    def start(self):
        self.before = gpu_clocks()
        self._thread.start()

    def stop(self):
        self._stop.set()
        self._thread.join(timeout=30)
        self.after = gpu_clocks()

    def summary(self):
        during = sorted(self.samples)
        return {"before": self.before, "after": self.after,
                "during_gfx_mean": ({"n": len(during), "min": during[0], "median": during[len(during) // 2],
                                     "max": during[-1]} if during else None)}


def copy_probe(mib, dev):
    """One device copy of mib MiB (mib MiB read, mib MiB written): the reference dispatch against which
    a profiler's HBM byte counters are calibrated in the same run."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy probe: {mib} MiB read + {mib} MiB written", file=sys.stderr)
    del src, dst


def bench_ffn(args):
    """The blockwise feed-forward on one device's share of the 1M-token context (131072 tokens of the
    1024-wide model, LLaMA's d_ff rule: 8/3 * 1024 rounded up to a multiple of 256 = 2816)."""
    import torch

    import long_context_exact_attn_amd as ra
    from long_context_exact_attn_amd import metrics as M
    T, d, f, chunk = 131072, 1024, 2816, args.ffn_chunk
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    x = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    w1 = (torch.randn((f, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    w3 = (torch.randn((f, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    w2 = (torch.randn((d, f), generator=g, device=dev) / f ** 0.5).to(torch.bfloat16)
    dout = torch.randn((T, d), generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(x)
    dx = torch.empty_like(x)
    dws = [torch.empty(w.shape, dtype=torch.float32, device=dev) for w in (w1, w3, w2)]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ra.blockwise_ffn_fwd(x, w1, w3, w2, chunk=chunk, out=out)
        if ev is not None:
            ev[1].record()
        ra.blockwise_ffn_bwd(x, w1, w3, w2, dout, chunk=chunk, dx=dx, dw1=dws[0], dw3=dws[1], dw2=dws[2])
        if ev is not None:
            ev[2].record()

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    unit = T * d * f
    fl_fwd, fl_bwd = 6 * unit, 12 * unit   # three products forward; six backward (recompute not counted)
    value = (fl_fwd + fl_bwd) / (ms_step * 1e-3) / 1e12
    kernels = {"ffn_fwd": {"ms": round(fwd_ms, 4), "tflops": round(fl_fwd / (fwd_ms * 1e-3) / 1e12, 2)},
               "ffn_bwd": {"ms": round(bwd_ms, 4), "tflops": round(fl_bwd / (bwd_ms * 1e-3) / 1e12, 2)}}
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    line = {"metric": "blockwise feed-forward TFLOP/s (fwd+bwd) at 1 MI355X", "value": round(value, 2),
            "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"blockwise SwiGLU feed-forward, 131072 tokens, d_model 1024, d_ff 2816, "
                                   f"chunks of {chunk} tokens", "pass": "fwd+bwd"},
            "frac_peak": round(value / M.PEAK_BF16_TFLOPS, 4), "kernels": kernels,
            "roofline": {"bound": "mfma", "kernel": dom, "achieved": kernels[dom]["tflops"],
                         "peak": M.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(kernels[dom]["tflops"] / M.PEAK_BF16_TFLOPS, 4), "traffic": None}}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the ring's K/V exchange across devices is not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.ffn:
        bench_ffn(args)
        return
    import torch

    import long_context_exact_attn_amd as ra
    from long_context_exact_attn_amd import metrics as M
    from long_context_exact_attn_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.ring_rank is not None:
        if w.ring_rank < 0 or not 0 <= args.ring_rank < w.n_ring:
            print(f"--ring-rank needs a one-rank workload and a rank in [0, {w.n_ring})", file=sys.stderr)
            sys.exit(2)
        w = W.replace(w, ring_rank=args.ring_rank, name=f"{w.name.rsplit('-r', 1)[0]}-r{args.ring_rank}")
    if args.ring_steps and not (w.ring_rank >= 0 and w.dtype == "bf16"):
        print("--ring-steps needs a one-rank bf16 workload", file=sys.stderr)
        sys.exit(2)
    if not w.backward and not args.fwd_only:
        w = W.replace(w, backward=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = W.make(w, device=dev)
    q, k, v, bias, seg = t["q"], t["k"], t["v"], t["bias"], t["segment_ids"]
    kw = dict(n_ring=w.n_ring, q_chunk=w.q_chunk, k_chunk=w.k_chunk, causal=w.causal, ring_rank=w.ring_rank)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.q_len), dtype=torch.float32, device=dev)
    if not args.fwd_only:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
    names = ["fwd"] if args.fwd_only else ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq"]
    if args.ring_steps and not args.fwd_only:
        names = ["fwd", "bwd_preprocess", "bwd_steps"]

    if args.ring_steps:
        # the blocks a device meets, in ring order, as contiguous receive buffers; causal blocks from
        # the future are not sent
        Lb, r, n = w.block_len, w.ring_rank, w.n_ring
        order = [(r - s_) % n for s_ in range(n)]
        order = [j for j in order if not (w.causal and j > r)]
        blocks = [(j, k[:, j * Lb:(j + 1) * Lb].contiguous(), v[:, j * Lb:(j + 1) * Lb].contiguous()) for j in order]
        B_, Lq_, H_, D_ = q.shape
        state = (torch.empty((B_, Lq_, H_, D_), dtype=torch.float32, device=dev),
                 torch.empty((B_, H_, Lq_), dtype=torch.float32, device=dev),
                 torch.empty((B_, H_, Lq_), dtype=torch.float32, device=dev))
        if not args.fwd_only:
            # dQ sums stay here; each block's dK / dV sums would travel on with it
            dq_acc = torch.empty((B_, Lq_, H_, D_), dtype=torch.float32, device=dev)
            dkv_acc = [(torch.empty_like(kb, dtype=torch.float32), torch.empty_like(vb, dtype=torch.float32))
                       for _, kb, vb in blocks]
            dkv_out = [(torch.empty_like(kb), torch.empty_like(vb)) for _, kb, vb in blocks]

    def forward():
        if not args.ring_steps:
            ra.blockwise_attn_fwd(q, k, v, bias, seg, out=out, lse=lse, **kw)
            return
        for i_, (j, kb, vb) in enumerate(blocks):
            ra.blockwise_attn_fwd_step(q, kb, vb, bias, seg, q_pos0=r * Lb, kv_pos0=j * Lb, causal=w.causal,
                                       state=state, init=i_ == 0)
        ra.blockwise_attn_fwd_finalize(state, out=out, lse=lse)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        forward()
        mark(1)
        if args.fwd_only:
            return
        ra.blockwise_attn_bwd_preprocess(out, t["dout"], delta=delta)
        mark(2)
        if args.ring_steps:
            for i_, (j, kb, vb) in enumerate(blocks):
                ra.blockwise_attn_bwd_step(q, kb, vb, lse, delta, t["dout"], bias, seg, q_pos0=r * Lb,
                                           kv_pos0=j * Lb, causal=w.causal, dq_acc=dq_acc, dk_acc=dkv_acc[i_][0],
                                           dv_acc=dkv_acc[i_][1], init_dq=i_ == 0, init_dkv=True)
            for i_ in range(len(blocks)):
                ra.blockwise_attn_bwd_finalize(dq_acc, *dkv_acc[i_], dq=dq, dk=dkv_out[i_][0], dv=dkv_out[i_][1])
            mark(3)
            return
        ra.blockwise_attn_bwd_dkdv(q, k, v, lse, delta, t["dout"], bias, seg, dk=dk, dv=dv, **kw)
        mark(3)
        ra.blockwise_attn_bwd_dq(q, k, v, lse, delta, t["dout"], bias, seg, dq=dq, **kw)
        mark(4)

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    clocks = ClockSampler()
    clocks.start()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clocks.stop()
    per = {n: sum(events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)) / args.steps
           for i, n in enumerate(names)}
    step_ms = sorted(events[s][0].elapsed_time(events[s][-1]) for s in range(args.steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                          step_ms[len(step_ms) // 2])
    ms_step = wall * 1e3 / args.steps

    segn = None if seg is None else seg.cpu().numpy()
    q_first = int(w.q_positions()[0]) if w.q_len else 0
    pairs = M.visible_pairs_per_head(q_first, w.q_len, w.kv_len, w.causal, segn)
    if segn is None:
        pairs *= w.batch
    fl = M.flops(pairs, w.head_dim, w.heads)
    # MFMA work the kernels execute: every tile a wave computes (masked and padding pairs included) at each
    # kernel's own tile shape; the dQ kernel's recomputation of S and dP included (dense masks only)
    ex = {}
    if segn is None and not args.ring_steps:
        D_, HB_ = w.head_dim, w.heads * w.batch
        if w.dtype == "bf16":
            nqb = 2 if w.head_dim == 64 else 1
            tiles = ((32 * nqb, 64), (128 if (w.head_dim == 64 and w.segments == "none") else 64, 32), (32, 64))
        else:   # the float32 kernels: 16 x 16 tiles throughout
            tiles = ((16, 16), (16, 16), (16, 16))
        e_fwd, e_kv, e_dq = (M.executed_pairs_per_head(q_first, w.q_len, w.kv_len, w.causal, tq, tk)
                             for tq, tk in tiles)
        if None not in (e_fwd, e_kv, e_dq):
            ex = {"fwd": 4 * D_ * e_fwd * HB_, "bwd_dkdv": 8 * D_ * e_kv * HB_, "bwd_dq": 6 * D_ * e_dq * HB_}
    kernel_flops = {"fwd": fl["fwd"], "bwd_dkdv": fl["dkdv"], "bwd_dq": fl["dq"], "bwd_steps": fl["dkdv"] + fl["dq"]}
    total_flops = fl["fwd"] if args.fwd_only else fl["fwd_bwd"]
    value = total_flops / (ms_step * 1e-3) / 1e12
    # a contraction is priced against the matrix unit's peak for its own dtype
    peak = M.PEAK_BF16_TFLOPS if w.dtype == "bf16" else M.PEAK_F32_TFLOPS
    kernels = {}
    for n in names:
        entry = {"ms": round(per[n], 4)}
        if n in kernel_flops:
            entry["tflops"] = round(kernel_flops[n] / (per[n] * 1e-3) / 1e12, 2)
            entry["frac_peak"] = round(entry["tflops"] / peak, 4)
        else:   # the preprocess streams out and dout once and writes delta
            nbytes = 2 * q.numel() * q.element_size() + lse.numel() * 4
            entry["gbs"] = round(nbytes / (per[n] * 1e-3) / 1e9, 1)
        kernels[n] = entry
    dom = max((n for n in names if n in kernel_flops), key=lambda n: per[n])
    ach = kernel_flops[dom] / (per[dom] * 1e-3) / 1e12
    fwd_tflops = fl["fwd"] / (per["fwd"] * 1e-3) / 1e12
    if ex:
        ex_total = ex["fwd"] if args.fwd_only else ex["fwd"] + ex["bwd_dkdv"] + ex["bwd_dq"]
        executed = {"tflops": round(ex_total / (ms_step * 1e-3) / 1e12, 2),
                    "flop_per_step": ex_total,
                    "per_kernel_tflops": {n: round(ex[n] / (per[n] * 1e-3) / 1e12, 2) for n in ex if n in per},
                    "note": "MFMA work executed: whole wave tiles, the dQ kernel's recomputed S and dP included "
                            "(18*D per pair for the step, against the 14*D counted in value)"}
    else:
        executed = None
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "ms_per_step_median": round(median_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: one device's share of a {w.kv_len}-token causal context "
                               f"(ring rank {w.ring_rank} of {w.n_ring}), {w.q_len} local queries, "
                               f"{w.heads} heads, head_dim {w.head_dim}" if w.ring_rank >= 0 else w.name,
                   "pass": ("fwd" if args.fwd_only else "fwd+bwd") + (" (ring steps)" if args.ring_steps else ""),
                   "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim, "q_len": w.q_len,
                   "kv_len": w.kv_len, "n_ring": w.n_ring, "ring_rank": w.ring_rank, "causal": w.causal,
                   "q_chunk": w.q_chunk, "k_chunk": w.k_chunk, "bias": w.bias_len > 0,
                   "segments": w.segments},
        "frac_peak": round(value / peak, 4),
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_frac_peak": round(fwd_tflops / peak, 4),
        "tokens_per_s": round(w.batch * w.q_len / (ms_step * 1e-3), 1),
        "visible_pairs": pairs * w.heads,
        "executed": executed,
        "clocks_mhz": clocks.summary(),
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                     "traffic": measured_traffic(w.name, dom)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, t, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
