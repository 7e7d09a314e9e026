"""Throughput of the compressed-KV decode path on one MI355X.

Workload (default): one GQA attention layer with 8 KV / 32 query heads,
head_dim 128, rank 32, 32K-token context, exact window 256, bf16 storage with
fp32 accumulation, batch 1; a block update + sync every 64 decode steps; keys
and values are a rank-32 Gaussian signal plus 1% noise (synthetic, seeded).

A step is one decode step of that layer: append one token (k, v) and decode
attention of 32 query heads over the whole mixed cache (one launch,
iskv_append_decode), plus the block updates (Brand fold of 64 tokens for all 8
heads, K and V) and coefficient syncs that fall due.  The bench holds 16
instances of the layer and runs the steps round-robin over them, as the
layers of one model decode a token (so every step reads its cache from HBM
rather than from the 256 MB Infinity Cache; one instance is ~35 MB).  All
instances fill their rings at the same token; by default (--fold-mode layers)
the step that completes that token folds every instance in one
iskv_block_update(-1) + iskv_sync(-1), as a multi-layer model would; with
--fold-mode instance each instance folds alone at its own step.

Prints one JSON line (see --help).  Only one GPU: --gpus N > 1 exits.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attn tokens/s + block updates/s; % of HBM roofline"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=512, help="untimed decode steps")
    ap.add_argument("--instances", type=int, default=16,
                    help="independent copies of the layer, stepped round-robin")
    ap.add_argument("--context", type=int, default=32768, help="tokens in the cache when timing starts")
    ap.add_argument("--rank", type=int, default=32)
    ap.add_argument("--rank-v", type=int, default=0,
                    help="rank of the V factor (0: same as --rank; else --rank or 2x --rank)")
    ap.add_argument("--window", type=int, default=256)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--fold-mode", choices=("layers", "instance"), default="layers",
                    help="layers: the instances are the layers of one model, and the token at which "
                         "they all fill their rings folds them in one block update + sync over every "
                         "layer (iskv_block_update(-1), iskv_sync(-1)); instance: each instance folds "
                         "alone at its own step")
    ap.add_argument("--protected-prefix", type=int, default=0,
                    help="leading positions kept exact and never folded (multiple of 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--async-maintenance", action="store_true",
                    help="run block updates and syncs on a second stream (each layer "
                         "instance's later work waits for its own); default: the decode stream")
    ap.add_argument("--ragged", action="store_true",
                    help="separate measurement: one layer, --batch sequences (default 16) whose "
                         "lengths are spread evenly up to --context; each step appends one token "
                         "to every sequence (iskv_append_ragged), attends each at its own length "
                         "(iskv_decode_attn_ragged), and folds the sequences whose ring fills")
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only stream a 256 MiB float32 tensor through an elementwise kernel "
                         "(x * 1 -> y) five times: the reference for HBM byte counters")
    return ap.parse_args()


def copy_calibration():
    """A plain streaming kernel of known traffic: reads and writes 256 MiB per
    dispatch.  HBM byte counters read on it give the scale factor between the
    counter and real bytes."""
    import torch
    n = 64 << 20
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "torch.mul(x, 1.0, out=y), float32", "dispatches": 5,
                      "bytes_read_per_dispatch": 4 * n, "bytes_written_per_dispatch": 4 * n}), flush=True)


def stream_bandwidth():
    """HBM bandwidth this GPU actually reaches on trivial streaming kernels
    (1 GiB float32): a read-only reduction (x.sum()) and a copy (y <- x, read
    + write bytes).  The best of ten dispatches each, timed by events on the
    current stream, outside the timed region; a second reference for the
    roofline next to the nominal 8 TB/s."""
    import torch
    n = 256 << 20
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    acc = torch.empty((), device="cuda")

    def best(fn, nbytes):
        fn()
        times = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b))
        return nbytes / (min(times) * 1e-3) / 1e9

    read = best(lambda: torch.sum(src, dim=0, out=acc), 4 * n)
    copy = best(lambda: dst.copy_(src), 8 * n)
    del src, dst
    return read, copy


# ---------------------------------------------------------------------------
# synthetic inputs (GPU-side generation, before the timed region)
# ---------------------------------------------------------------------------

class Generator:
    """x_t = G z_t + 0.01 e_t per (instance, KV head, K|V); G fixed, 128 x 32."""

    def __init__(self, torch, n_inst, batch, kv_heads, d, signal_rank, seed):
        self.torch = torch
        self.g = torch.Generator(device="cuda")
        self.g.manual_seed(seed)
        self.mix = torch.randn(n_inst, batch, kv_heads, 2, signal_rank, d, device="cuda",
                               generator=self.g) / math.sqrt(signal_rank)
        self.shape = (batch, kv_heads, d, signal_rank)

    def tokens(self, inst, n):
        torch = self.torch
        b, h, d, k = self.shape
        z = torch.randn(b, h, 2, n, k, device="cuda", generator=self.g)
        x = torch.matmul(z, self.mix[inst]) + 0.01 * torch.randn(b, h, 2, n, d, device="cuda",
                                                                generator=self.g)
        x = x.permute(2, 0, 3, 1, 4).contiguous()          # [2, b, n, h, d]
        return x[0], x[1]

    def queries(self, count, q_heads, d):
        return self.torch.randn(count, self.shape[0], q_heads, d, device="cuda", generator=self.g)


def decode_bytes(batch, kv_heads, q_heads, d, r, n_c, n_e, elem=2, r_v=None):
    """Algorithmic bytes of one decode call: coefficients of K (rank r) and V
    (rank r_v, default r), exact window rows of K and V, the two fp32 bases,
    the fp32 query and output."""
    rs = r + (r_v or r)
    per_unit = n_c * rs * elem + n_e * d * 2 * elem + d * rs * 4
    return batch * kv_heads * per_unit + batch * q_heads * d * 4 * 2


def kernel_source_hash():
    h = hashlib.sha256()
    src = os.path.join(ROOT, "rank_decode_attention_iskv_amd", "csrc")
    for name in sorted(os.listdir(src)):
        with open(os.path.join(src, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_hash):
    """Per-launch HBM bytes of the decode kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "decode_attn_r32_ctx32k_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.strip().split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores, bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(context, window, rank, kv_heads, q_heads, decode_queries=4):
    from threadpoolctl import threadpool_limits

    # the oracle is plain numpy; its BLAS calls are held to one thread so the
    # figure is per core and reproducible
    with threadpool_limits(limits=1):
        return _cpu_baseline(context, window, rank, kv_heads, q_heads, decode_queries)


def _cpu_baseline(context, window, rank, kv_heads, q_heads, decode_queries, sample_heads=3):
    import workloads
    from oracle import Unit

    cores = 1
    w = workloads.with_(workloads.WORKLOADS[2], window=window, rank=rank, context=context)
    units = [Unit(w.head_dim, rank, window, context + 64, "bf16") for _ in range(sample_heads)]
    t0 = time.perf_counter()
    fold_t = 0.0
    folds = 0
    pos = 0
    while pos < context:
        n = min(64, context - pos)
        k, v = workloads.tokens(w, 0, pos, n)
        for h, u in enumerate(units):
            for i in range(n):
                u.append(k[0, i, h], v[0, i, h])
        pos += n
        for u in units:
            if u.ready:
                f0 = time.perf_counter()
                u.fold()
                u.sync()
                fold_t += time.perf_counter() - f0
                folds += 1
    build_t = time.perf_counter() - t0
    g = q_heads // kv_heads
    d0 = time.perf_counter()
    for s in range(decode_queries):
        q = workloads.query(w, 0, s)[0]
        for h, u in enumerate(units):
            u.decode(q[h * g:(h + 1) * g], u.length - 1, 1.0 / math.sqrt(w.head_dim))
    dec_t = (time.perf_counter() - d0) / (decode_queries * sample_heads)
    # one decode step of the layer: kv_heads units decode; every 64 steps each
    # unit folds + syncs at the current history length (averaged over the
    # sample's whole growth to `context`)
    fold_avg = fold_t / max(folds, 1)
    step_s = kv_heads * (dec_t + fold_avg / 64.0)
    return {
        "value": 1.0 / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"{sample_heads} KV heads (K and V each) of the layer built to {context} tokens by the "
                   f"float64 oracle ({folds} folds + syncs, {build_t:.1f} s), then {decode_queries} decode "
                   f"calls of {g} query heads per KV head ({dec_t * 1e3:.1f} ms each); one step = "
                   f"{kv_heads} KV heads x (decode + average fold+sync / 64); BLAS held to one thread"),
        "oracle_decode_ms_per_head": dec_t * 1e3,
        "oracle_fold_sync_ms_avg": fold_avg * 1e3,
    }


def ragged_bench(args):
    """A ragged batch: sequence b holds about context * (b + 1) / B tokens."""
    import torch

    from rank_decode_attention_iskv_amd import binding
    torch.cuda.set_device(0)
    H, HQ, D, R, W = 8, 32, 128, args.rank, args.window
    B = args.batch if args.batch > 1 else 16
    RV = args.rank_v or R
    target = [max(1, args.context * (b + 1) // B) for b in range(B)]
    steps = args.warmup + args.steps
    cfg = binding.make_config(B, 1, H, HQ, D, R, W, args.context + steps + 64, binding.BF16,
                              protected_prefix=args.protected_prefix, rank_v=RV)
    cache = binding.IskvCache(cfg)
    gen = Generator(torch, 1, B, H, D, 32, args.seed)
    slots = W + 64
    length, n_c = [0] * B, [args.protected_prefix] * B
    t_pre = time.perf_counter()
    while any(length[b] < target[b] for b in range(B)):
        counts = [max(0, min(64, target[b] - length[b], slots - (length[b] - n_c[b]))) for b in range(B)]
        k, v = gen.tokens(0, max(counts))
        ready = cache.append_ragged(0, k, v, counts)
        for b in range(B):
            length[b] += counts[b]
        if ready:
            cache.block_update(0)
            cache.sync(0)
            for b in range(B):
                if length[b] - n_c[b] == slots:
                    n_c[b] += 64
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t_pre
    toks = [gen.tokens(0, 1) for _ in range(steps)]
    q_all = gen.queries(steps, HQ, D)
    out = torch.empty(B, HQ, D, device="cuda")
    ones = [1] * B
    folds = 0

    def step(s):
        nonlocal folds
        k, v = toks[s]
        ready = cache.append_ragged(0, k, v, ones)
        for b in range(B):
            length[b] += 1
        cache.decode_attn_ragged(0, q_all[s], [L - 1 for L in length], out)
        if ready:
            cache.block_update(0)
            cache.sync(0)
            folds += 1
            for b in range(B):
                if length[b] - n_c[b] == slots:
                    n_c[b] += 64

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, steps):
        step(s)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    # decode roofline: back-to-back ragged decode calls at the final lengths
    calls = 64
    rl_bytes = sum(decode_bytes(1, H, HQ, D, R, n_c[b] - args.protected_prefix,
                                length[b] - (n_c[b] - args.protected_prefix), r_v=RV)
                   for b in range(B))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qp = [L - 1 for L in length]
    e0.record(stream)
    for _ in range(calls):
        cache.decode_attn_ragged(0, q_all[0], qp, out)
    e1.record(stream)
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / calls
    achieved = rl_bytes / (avg_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC + " (ragged batch)",
        "value": B * args.steps / total_s,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_s * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": (f"one GQA layer, ragged batch of {B} sequences at lengths "
                         f"{target[0]}..{target[-1]} (spread evenly), {H} KV / {HQ} q heads, "
                         f"head_dim {D}, rank {R} (V {RV}), window {W}, bf16 storage; per step one "
                         "token per sequence (iskv_append_ragged), iskv_decode_attn_ragged, and a "
                         "fold + sync of the sequences whose ring fills"),
            "global_batch": B, "seq_len": args.context, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_attn_ragged", "achieved": achieved, "peak": 8000.0,
            "unit": "GB/s", "frac": achieved / 8000.0, "traffic": None,
            "algorithmic_bytes_per_launch": rl_bytes, "avg_launch_us": avg_ms * 1e3,
        },
        "cpu_baseline": None,
        "folds_timed": folds, "prefill_s": t_pre,
    }
    print(json.dumps(res))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); runs over several "
              "GPUs are not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ragged:
        ragged_bench(args)
        return
    import torch

    from rank_decode_attention_iskv_amd import binding

    torch.cuda.set_device(0)
    H, HQ, D, R, W, B = 8, 32, 128, args.rank, args.window, args.batch
    I = args.instances
    total_steps = args.warmup + args.steps
    per_inst_steps = (total_steps + I - 1) // I
    max_tokens = args.context + per_inst_steps + 64
    P = args.protected_prefix
    RV = args.rank_v or R
    cfg = binding.make_config(B, I, H, HQ, D, R, W, max_tokens, binding.BF16, protected_prefix=P,
                              rank_v=RV)
    cache = binding.IskvCache(cfg)
    stream = torch.cuda.current_stream()
    gen = Generator(torch, I, B, H, D, 32, args.seed)

    # ---- prefill every instance to `context` tokens (fold + sync as the ring fills)
    t_pre = time.perf_counter()
    length, n_c = 0, 0
    while length < args.context:
        n = min(64, args.context - length, (W + 64) - (length - P - n_c))
        ready = False
        for inst in range(I):
            k, v = gen.tokens(inst, n)
            ready = cache.append(inst, k, v)
        length += n
        if ready:
            cache.block_update(-1)
            cache.sync(-1)
            n_c += 64
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t_pre

    # ---- inputs of the timed steps, resident before timing
    # per instance [step][batch][1][kv_heads][d], so each step's token is one
    # contiguous [batch, 1, kv_heads, d] block
    k_all, v_all = [], []
    for inst in range(I):
        k, v = gen.tokens(inst, per_inst_steps)            # [B, n, H, D]
        k_all.append(k.permute(1, 0, 2, 3).contiguous())
        v_all.append(v.permute(1, 0, 2, 3).contiguous())
    q_all = gen.queries(total_steps, HQ, D)
    out = torch.empty(B, HQ, D, device="cuda")
    torch.cuda.synchronize()

    lengths = [cache.status(i).length for i in range(I)]
    comp = [cache.status(i).compressed for i in range(I)]
    used = [0] * I
    ev = []                      # (start, end, bytes) per timed decode launch
    mstream = None
    fold_ev, sync_ev = [], []
    bytes_total = 0
    folds = 0
    n_ready = 0                  # instances whose ring is full (fold mode "layers")

    # The step loop calls the C ABI directly with precomputed device pointers
    # and pre-created events: the per-step host work must stay well below the
    # GPU time of a step, or the timeline measures the Python loop.
    import ctypes
    L_ = binding.lib()
    ctx = cache.ctx
    tok_bytes = B * H * D * 4
    k_base = [t.data_ptr() for t in k_all]
    v_base = [t.data_ptr() for t in v_all]
    q_base, q_bytes = q_all.data_ptr(), B * HQ * D * 4
    out_p = ctypes.c_void_p(out.data_ptr())
    ready_c = ctypes.c_int(0)
    ev_pool = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.warmup)]

    def step(s, timed, warm=False):
        nonlocal bytes_total, folds, mstream, n_ready
        inst = s % I
        j = used[inst]
        used[inst] += 1
        lengths[inst] += 1
        L, n_c = lengths[inst], comp[inst]
        kp = ctypes.c_void_p(k_base[inst] + j * tok_bytes)
        vp = ctypes.c_void_p(v_base[inst] + j * tok_bytes)
        qp = ctypes.c_void_p(q_base + s * q_bytes)
        # append + decode attention of the step in one launch (iskv_append_decode);
        # warm-up steps carry an event pair around it, timed steps carry none
        if warm:
            e0, e1 = ev_pool[len(ev)]
            e0.record(stream)
            code = L_.iskv_append_decode(ctx, inst, kp, vp, binding.F32, qp, L - 1, out_p,
                                         ctypes.byref(ready_c))
            e1.record(stream)
            ev.append((e0, e1, decode_bytes(B, H, HQ, D, R, n_c, L - n_c, r_v=RV)))
        else:
            code = L_.iskv_append_decode(ctx, inst, kp, vp, binding.F32, qp, L - 1, out_p,
                                         ctypes.byref(ready_c))
            bytes_total += decode_bytes(B, H, HQ, D, R, n_c, L - n_c, r_v=RV)
        if code != 0:
            raise binding.IskvError(code, "iskv_append_decode")
        ready = bool(ready_c.value)
        if not ready:
            return
        comp[inst] += 64
        if args.fold_mode == "layers":
            # every instance (layer) fills its ring at the same token; the
            # last one's step folds them all in one launch pair
            n_ready += 1
            if n_ready < I:
                return
            n_ready = 0
            layer, nfold = -1, I
        else:
            layer, nfold = inst, 1
        if warm or (timed and (not args.async_maintenance)):
            f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            f0.record(stream)
            cache.block_update(layer)
            f1.record(stream)
            cache.sync(layer)
            f2.record(stream)
            fold_ev.append((f0, f1))
            sync_ev.append((f1, f2))
        else:
            cache.block_update(layer)
            cache.sync(layer)
        folds += 0 if warm else nfold

    # warm-up on one stream, with the fold and sync kernels timed by events
    for s in range(args.warmup):
        step(s, True, warm=True)
    torch.cuda.synchronize()
    if args.async_maintenance:
        mstream = torch.cuda.Stream()
        cache.set_maintenance_stream(mstream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.warmup, total_steps):
        step(s, True)
    if mstream is not None:
        cache.join_maintenance()          # the timed region ends after every fold and sync
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    dec_ms = [a.elapsed_time(b) for a, b, _ in ev]          # warm-up steps only
    dec_avg_ms = sum(dec_ms) / len(dec_ms) if dec_ms else None

    # ---- roofline of the decode kernel: one event pair around back-to-back
    # decode calls over the instances at their final lengths (the per-step
    # event pairs above also hold the dispatch gap before each kernel)
    rl_calls = max(4 * I, 64)
    rl_bytes = 0
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qp = ctypes.c_void_p(q_base)
    r0.record(stream)
    for c in range(rl_calls):
        inst = c % I
        code = L_.iskv_decode_attn(ctx, inst, qp, lengths[inst] - 1, out_p)
        if code != 0:
            raise binding.IskvError(code, "iskv_decode_attn")
        rl_bytes += decode_bytes(B, H, HQ, D, R, comp[inst], lengths[inst] - comp[inst], r_v=RV)
    r1.record(stream)
    torch.cuda.synchronize()
    rl_avg_ms = r0.elapsed_time(r1) / rl_calls
    bytes_avg = rl_bytes / rl_calls
    achieved = bytes_avg / (rl_avg_ms * 1e-3) / 1e9
    fold_ms = [a.elapsed_time(b) for a, b in fold_ev]
    sync_ms = [a.elapsed_time(b) for a, b in sync_ev]
    units_per_fold = B * H * 2
    layers_per_launch = I if args.fold_mode == "layers" else 1
    st = cache.status(0)
    flags = max(cache.status(i).numeric_flags for i in range(I))
    finite = bool(torch.isfinite(out).all().item())
    value = args.steps / (total_ms * 1e-3)
    kh = kernel_source_hash()
    traffic = committed_traffic(kh)
    bw_read, bw_copy = stream_bandwidth()

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"one GQA layer: {H} KV / {HQ} q heads, head_dim {D}, rank {R}, "
                         f"{args.context}-token context (grows by 1 per step), window {W}, "
                         f"bf16 storage, fp32 accumulate, batch {B}, block update + sync every "
                         f"64 tokens; K/V rank-32 signal + 1% noise"
                         + (f"; first {P} positions kept exact (protected prefix)" if P else "")
                         + (f"; V rank {RV}" if RV != R else "")),
            "protected_prefix": P,
            "rank_v": RV,
            "instances_rotated": I,
            "global_batch": B,
            "seq_len": args.context,
            "parallelism": "single GPU",
            "step_calls": ("iskv_append_decode; every 64 tokens iskv_block_update(-1) + iskv_sync(-1) "
                           f"over all {I} instances (layers) at once" if args.fold_mode == "layers" else
                           "iskv_append_decode; every 64 steps per instance iskv_block_update + iskv_sync"),
            "fold_mode": args.fold_mode,
            "maintenance": "same stream" if (not args.async_maintenance) else
                           "second stream (each instance waits for its own fold + sync)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_attn",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_avg,
            "avg_launch_us": rl_avg_ms * 1e3,
            "launches_timed": rl_calls,
            "avg_launch_us_in_step": dec_avg_ms * 1e3 if dec_avg_ms else None,
            "measured_stream_read_GBs": bw_read,
            "measured_stream_copy_GBs": bw_copy,
            "frac_of_measured_read": achieved / bw_read,
        },
        "decode_attn_calls_per_s_kernel_only": 1e3 / rl_avg_ms,
        "block_updates_per_s": (units_per_fold * layers_per_launch * len(fold_ms) / (sum(fold_ms) * 1e-3))
                               if fold_ms else None,
        "block_updates_per_s_with_sync": (units_per_fold * layers_per_launch * len(fold_ms) /
                                          ((sum(fold_ms) + sum(sync_ms)) * 1e-3)) if fold_ms else None,
        "fold_launch_layers": layers_per_launch,
        "fold_avg_us": (sum(fold_ms) / len(fold_ms) * 1e3) if fold_ms else None,
        "sync_avg_us": (sum(sync_ms) / len(sync_ms) * 1e3) if sync_ms else None,
        "timed_folds": folds,
        "prefill_s": t_pre,
        "wall_s_timed": wall,
        "numeric_flags": flags,
        "output_finite": finite,
        "kernel_sources_sha256_16": kh,
        "persistent_kv_bytes_per_instance": st.persistent_bytes // I,
        "full_kv_bytes_per_instance": st.full_bytes // I,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.context, W, R, H, HQ)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
