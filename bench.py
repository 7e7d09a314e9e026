"""Throughput of the compressed-KV decode path on one MI355X.

Five workloads (--config 1..5, default 3):

  1  1 KV / 1 query head, head_dim 128, rank 32, 4,096-token context, window
     256, fp32 storage; keys/values rank-24 Gaussian signal + 1% noise
  2  one GQA layer: 8 KV / 32 query heads, rank 32, 32K context, window 256,
     bf16 storage, batch 1; rank-32 signal + 1% noise
  3  batch 16 x 16K context, 8 KV / 32 query heads, rank 64, window 512, bf16;
     spectra decaying as sigma_i ~ 1/i, per-sequence bases
  4  36 layers x 8 KV / 32 query heads, rank 32, window 1,024, bf16, 64K
     context (--context: any point of the 4K -> 64K growth); 30% of old keys
     high-norm and aligned with the later queries
  5  batch 64 x 8K context, 8 KV / 32 query heads, bf16, one point of the sweep
     rank {16,32,64,128} x window {128,1024} (--rank, --window; default 32/128)

A step is one decode step of the whole model of the workload (one layer for
1, 2, 3 and 5; 36 layers for 4) for every sequence of the batch: append the
new token's k, v and attend with every query head over the whole mixed cache
(iskv_append_decode, one launch per layer), plus the block updates (Brand
fold of the 64 tokens that left the window, every unit, K and V) and the
syncs (rewrite of every older coefficient row) that fall due, one fold event
per 64 steps.  Inputs are synthetic, seeded and resident in HBM before
timing.  Workloads whose cache is smaller than 512 MB keep several
instances of the model (--instances) and step them round-robin, so that
every step reads its cache from HBM and not from the 256 MB Infinity Cache.

Timing (HIP events on the launch stream): the timed steps run in segments of
decode steps; each fold event that falls due between segments (block update
+ sync of every layer whose ring is full, all instances at once) is timed by
its own event pair, and at least two fold events are timed per run (extra
ones after the steps if the steps hold fewer).  ms_per_step = decode time
per step + the fold event time amortized at its natural rate (one event per
64 steps of every instance); value = tokens per second of the whole batch.

The default run (config 3) also reports config 2 and the config-5 sweep
points as extra keys (--no-extras skips them), and the float64 oracle timed
on the host cores (cpu_baseline; --no-cpu-baseline skips it).

Prints one JSON line.  Only one GPU: --gpus N > 1 exits.
"""

from __future__ import annotations

import argparse
import ctypes
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
ROTATE_BYTES = 512 << 20

# workload presets: storage 0 = fp32, 1 = bf16
PRESETS = {
    1: dict(batch=1, layers=1, kv=1, q=1, rank=32, window=256, context=4096, storage=0,
            spectrum="gauss", signal=24, hot=0.0),
    2: dict(batch=1, layers=1, kv=8, q=32, rank=32, window=256, context=32768, storage=1,
            spectrum="gauss", signal=32, hot=0.0),
    3: dict(batch=16, layers=1, kv=8, q=32, rank=64, window=512, context=16384, storage=1,
            spectrum="power", signal=128, hot=0.0),
    4: dict(batch=1, layers=36, kv=8, q=32, rank=32, window=1024, context=65536, storage=1,
            spectrum="gauss", signal=32, hot=0.3),
    5: dict(batch=64, layers=1, kv=8, q=32, rank=32, window=128, context=8192, storage=1,
            spectrum="gauss", signal=32, hot=0.0),
}
SWEEP5 = [(r, w) for r in (16, 32, 64, 128) for w in (128, 1024)]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", type=int, default=3, choices=sorted(PRESETS))
    ap.add_argument("--steps", type=int, default=256, help="timed decode steps")
    ap.add_argument("--warmup", type=int, default=32, help="untimed decode steps")
    ap.add_argument("--instances", type=int, default=0,
                    help="copies of the model stepped round-robin (0: enough for 512 MB of cache)")
    ap.add_argument("--context", type=int, default=0, help="tokens in the cache when timing starts")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--rank-v", type=int, default=0,
                    help="rank of the V factor (0: same as --rank; else --rank or 2x --rank)")
    ap.add_argument("--window", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0)
    ap.add_argument("--protected-prefix", type=int, default=0,
                    help="leading positions kept exact and never folded (multiple of 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default config only: skip the config-2 and config-5 extra keys")
    ap.add_argument("--ragged", action="store_true",
                    help="separate measurement: one layer, --batch sequences (default 16) whose "
                         "lengths are spread evenly up to --context; each step appends one token "
                         "to every sequence (iskv_append_ragged), attends each at its own length "
                         "(iskv_decode_attn_ragged), and folds the sequences whose ring fills")
    ap.add_argument("--seed", type=int, default=1000)
    ap.add_argument("--joint-heads", action="store_true",
                    help="one basis per (sequence, layer) over all KV heads (joint_heads = 1); "
                         "the heads' inputs mix shared latent factors")
    ap.add_argument("--async-maintenance", action="store_true",
                    help="copy-on-write maintenance on a second stream (iskv_maintain / "
                         "iskv_switch) instead of block update + sync between decode steps")
    ap.add_argument("--prefill", action="store_true",
                    help="only compare prefill paths: a 32K prompt into 16 layers of the "
                         "32K GQA workload, block by block vs iskv_prefill_layers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only stream a 256 MiB float32 tensor through an elementwise kernel "
                         "(x * 1 -> y) five times: the reference for HBM byte counters")
    return ap.parse_args()


def preset(args, cfg_id=None, **over):
    p = dict(PRESETS[cfg_id or args.config])
    for k, a in (("context", "context"), ("rank", "rank"), ("window", "window"), ("batch", "batch")):
        v = getattr(args, a) if cfg_id is None else 0
        if v:
            p[k] = v
    p["rank_v"] = (args.rank_v if cfg_id is None else 0) or p["rank"]
    p["prefix"] = args.protected_prefix if cfg_id is None else 0
    p["joint"] = int(args.joint_heads) if cfg_id is None else 0
    p.update(over)
    p["id"] = cfg_id or args.config
    return p


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
    """HBM bandwidth of a plain copy (y <- x, 1 GiB float32, read + write
    bytes), best of ten dispatches timed by events: a second reference for
    the roofline next to the nominal 8 TB/s."""
    import torch
    n = 256 << 20
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    times = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 8 * n / (min(times) * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# synthetic inputs (GPU-side generation, before the timed region)
# ---------------------------------------------------------------------------

class Generator:
    """Per (instance-layer, sequence, KV head, K|V): x_t = G diag(s) z_t + 0.01 e_t
    with G Gaussian (d x k, "gauss") or Haar-orthonormal columns with s_i ~ 1/i
    ("power"); with hot > 0 a Bernoulli share of keys gets + 4 sqrt(d) u, u a unit
    vector per (layer, KV head), and queries get + 2 u.  Joint-head presets draw
    z_t once per (sequence, K|V) for all heads."""

    def __init__(self, torch, p, n_layers, seed):
        self.torch, self.p = torch, p
        self.g = torch.Generator(device="cuda")
        self.g.manual_seed(seed)
        B, H, d, k = p["batch"], p["kv"], 128, p["signal"]
        shape = (n_layers, B, H, 2)
        if p["spectrum"] == "power":
            # Haar-orthonormal columns: QR of a Gaussian matrix, on the host
            # (a device QR is a library call the profilers' counter mode can fail in)
            z = torch.randn(*shape, d, d, device="cuda", generator=self.g)
            o, _ = torch.linalg.qr(z.cpu())
            o = o.cuda()
            s = 1.0 / torch.arange(1, k + 1, device="cuda", dtype=torch.float32)
            s = s * math.sqrt(d / float((s ** 2).sum()))
            self.mix = (o[..., :k] * s).transpose(-1, -2).contiguous()       # [.., k, d]
            self.noise = 0.0
        else:
            self.mix = torch.randn(*shape, k, d, device="cuda", generator=self.g) / math.sqrt(k)
            self.noise = 0.01
        u = torch.randn(n_layers, H, d, device="cuda", generator=self.g)
        self.hot_dir = u / u.norm(dim=-1, keepdim=True)

    def tokens(self, layer, n):
        """k, v: [batch, n, kv_heads, d] float32."""
        torch, p = self.torch, self.p
        B, H, d, k = p["batch"], p["kv"], 128, p["signal"]
        if p.get("joint"):
            # the heads of a sequence mix the same latent factors
            z = torch.randn(B, 1, 2, n, k, device="cuda", generator=self.g).expand(B, H, 2, n, k)
        else:
            z = torch.randn(B, H, 2, n, k, device="cuda", generator=self.g)
        x = torch.matmul(z, self.mix[layer])
        if self.noise:
            x = x + self.noise * torch.randn(B, H, 2, n, d, device="cuda", generator=self.g)
        if p["hot"] > 0:
            hot = (torch.rand(B, H, n, 1, device="cuda", generator=self.g) < p["hot"]).float()
            x[:, :, 0] += hot * (4.0 * math.sqrt(d)) * self.hot_dir[layer][None, :, None, :]
        x = x.permute(2, 0, 3, 1, 4).contiguous()          # [2, B, n, H, d]
        return x[0], x[1]

    def queries(self, count, layer):
        torch, p = self.torch, self.p
        q = torch.randn(count, p["batch"], p["q"], 128, device="cuda", generator=self.g)
        if p["hot"] > 0:
            g = p["q"] // p["kv"]
            q += 2.0 * self.hot_dir[layer].repeat_interleave(g, dim=0)[None, None]
        return q


def decode_bytes(p, n_c, n_e):
    """Algorithmic bytes of one decode call of one layer: coefficients of K
    (rank r) and V (rank r_v) -- per KV head, or once per sequence with a
    joint basis --, the exact rows of K and V (window ring and protected
    prefix), the two fp32 bases, the fp32 query and output."""
    elem = 2 if p["storage"] == 1 else 4
    rs = p["rank"] + p["rank_v"]
    coef = n_c * rs * elem
    per_unit = n_e * 128 * 2 * elem + 128 * rs * 4 + (0 if p.get("joint") else coef)
    seq = coef if p.get("joint") else 0
    return p["batch"] * (p["kv"] * per_unit + seq) + p["batch"] * p["q"] * 128 * 4 * 2


def state_bytes(p, n_c, n_e):
    elem = 2 if p["storage"] == 1 else 4
    coef = n_c * (p["rank"] + p["rank_v"]) * elem
    heads = p["kv"] * n_e * 256 * elem
    return p["layers"] * p["batch"] * ((coef if p.get("joint") else coef * p["kv"]) + heads)


DECODE_SOURCES = ("decode.hip", "device_common.hpp", "iskv_internal.hpp")


def kernel_source_hash():
    """Hash of the decode kernel's sources (the kernel the roofline and the
    committed counter summaries describe)."""
    h = hashlib.sha256()
    src = os.path.join(ROOT, "rank_decode_attention_iskv_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(src, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_hash, p):
    """Per-launch HBM bytes of the decode kernel from the committed rocprofv3
    counter summary of this workload, if taken on the current kernel sources."""
    tag = f"_joint_r{p['rank']}" if p.get("joint") else ""
    path = os.path.join(ROOT, "profiles", f"decode_attn_config{p['id']}{tag}_counters.txt")
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


def describe(p):
    names = {1: "1 KV / 1 query head", 2: "one GQA layer, 8 KV / 32 query heads",
             3: "8 KV / 32 query heads", 4: "36 layers x 8 KV / 32 query heads",
             5: "8 KV / 32 query heads"}
    sig = ("sigma_i ~ 1/i spectra" if p["spectrum"] == "power" else
           f"rank-{p['signal']} signal + 1% noise")
    s = (f"config {p['id']}: batch {p['batch']} x {p['context']}-token context (grows by 1 per "
         f"step), {names[p['id']]}, head_dim 128, rank {p['rank']}"
         + (f" (V {p['rank_v']})" if p["rank_v"] != p["rank"] else "")
         + f", window {p['window']}, {'bf16' if p['storage'] == 1 else 'fp32'} storage, fp32 "
         f"accumulate; K/V {sig}"
         + ("; 30% hot keys aligned with the queries" if p["hot"] else "")
         + (f"; first {p['prefix']} positions exact" if p["prefix"] else "")
         + ("; one basis per sequence over the 8 KV heads (joint), heads mixing shared latent "
            "factors" if p.get("joint") else "")
         + "; block update + sync every 64 tokens")
    return s


# ---------------------------------------------------------------------------
# one workload: prefill, timed steps, fold events, roofline
# ---------------------------------------------------------------------------

def measure(p, steps, warmup, instances, seed, quiet=False):
    import torch

    from rank_decode_attention_iskv_amd import binding
    torch.cuda.set_device(0)
    L0, W, P, ML = p["context"], p["window"], p["prefix"], p["layers"]
    slots = W + 64
    # the compressed count that leaves W exact tokens at L0 (fold events
    # happen at the token that fills the rings)
    n_c0 = max(P, (L0 - W - P) // 64 * 64 + P)
    n_e0 = L0 - n_c0
    if instances <= 0:
        instances = max(1, math.ceil(ROTATE_BYTES / max(1, state_bytes(p, n_c0 - P, n_e0))))
    I = min(instances, 64)
    nl = I * ML
    per_inst = (warmup + steps + I - 1) // I
    max_tokens = L0 + per_inst + 64 * 3 + 64
    cfg = binding.make_config(p["batch"], nl, p["kv"], p["q"], 128, p["rank"], W, max_tokens,
                              p["storage"], protected_prefix=P, rank_v=p["rank_v"],
                              joint_heads=p.get("joint", 0))
    cache = binding.IskvCache(cfg)
    stream = torch.cuda.current_stream()
    gen = Generator(torch, p, nl, seed)

    # ---- prefill every layer of every instance to L0 (fold + sync as the rings fill)
    t_pre = time.perf_counter()
    length, n_c = 0, P
    while length < L0:
        n = min(256, L0 - length, slots - (length - n_c) if length >= P else P - length)
        ready = False
        for layer in range(nl):
            k, v = gen.tokens(layer, n)
            ready = cache.append(layer, k, v)
        length += n
        if ready:
            cache.block_update(-1)
            cache.sync(-1)
            n_c += 64
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t_pre
    if not quiet:
        print(f"# config {p['id']}: {nl} layers prefilled to {length} tokens in {t_pre:.1f} s",
              file=sys.stderr, flush=True)

    # ---- inputs of every step, resident before timing: per layer
    # [step][batch][1][kv][d], one contiguous block per step
    B, H, HQ = p["batch"], p["kv"], p["q"]
    tok_bytes = B * H * 128 * 4
    need = per_inst + 64 * 3
    k_all, v_all = [], []
    for layer in range(nl):
        k, v = gen.tokens(layer, need)
        k_all.append(k.permute(1, 0, 2, 3).contiguous())
        v_all.append(v.permute(1, 0, 2, 3).contiguous())
    q_all = [gen.queries(per_inst, layer) for layer in range(ML)]
    q_bytes = B * HQ * 128 * 4
    out = torch.empty(B, HQ, 128, device="cuda")
    torch.cuda.synchronize()

    lib = binding.lib()
    ctx = cache.ctx
    k_base = [t.data_ptr() for t in k_all]
    v_base = [t.data_ptr() for t in v_all]
    q_base = [t.data_ptr() for t in q_all]
    out_p = ctypes.c_void_p(out.data_ptr())
    ready_c = ctypes.c_int(0)
    lens = [length] * nl            # per layer
    comp = [n_c] * nl
    used = [0] * nl
    n_ready = [0]
    fold_ms, sync_ms = [], []
    bytes_steps = [0]

    def fold_event():
        f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        f0.record(stream)
        cache.block_update(-1)
        f1.record(stream)
        cache.sync(-1)
        f2.record(stream)
        return f0, f1, f2

    events = []

    def step(s):
        """Decode step s: instance s % I, every layer of it.  Returns True if
        the step completed the token that fills every instance's rings."""
        inst = s % I
        due = False
        for l in range(ML):
            layer = inst * ML + l
            j = used[layer]
            used[layer] += 1
            lens[layer] += 1
            L = lens[layer]
            code = lib.iskv_append_decode(ctx, layer, ctypes.c_void_p(k_base[layer] + j * tok_bytes),
                                          ctypes.c_void_p(v_base[layer] + j * tok_bytes), binding.F32,
                                          ctypes.c_void_p(q_base[l] + (s // I) * q_bytes), L - 1,
                                          out_p, ctypes.byref(ready_c))
            if code != 0:
                raise binding.IskvError(code, "iskv_append_decode")
            bytes_steps[0] += decode_bytes(p, comp[layer] - P, L - (comp[layer] - P))
            if ready_c.value:
                comp[layer] += 64
                n_ready[0] += 1
        if n_ready[0] == nl:
            n_ready[0] = 0
            due = True
        return due

    # warm-up: untimed steps, folds as they fall due
    for s in range(warmup):
        if step(s):
            cache.block_update(-1)
            cache.sync(-1)
    torch.cuda.synchronize()
    bytes_steps[0] = 0

    # timed steps in segments; fold events between segments, timed alone
    segs = []
    s = warmup
    wall0 = time.perf_counter()
    while s < warmup + steps:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        due = False
        while s < warmup + steps and not due:
            due = step(s)
            s += 1
        e1.record(stream)
        segs.append((e0, e1))
        if due:
            events.append(fold_event())
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    timed_folds = len(events)
    # at least two fold events per run: fill the rings (untimed appends of the
    # prepared tokens) and fold
    while len(events) < 2:
        for layer in range(nl):
            room = slots - (lens[layer] - (comp[layer] - P) - P) if lens[layer] >= P else 0
            if room > 0:
                j = used[layer]
                kk = k_all[layer][j: j + room].permute(1, 0, 2, 3).contiguous()
                vv = v_all[layer][j: j + room].permute(1, 0, 2, 3).contiguous()
                used[layer] += room
                lens[layer] += room
                cache.append(layer, kk, vv)
            comp[layer] += 64
        events.append(fold_event())
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in segs)
    fold_ms = [a.elapsed_time(b) for a, b, _ in events]
    sync_ms = [b.elapsed_time(c) for _, b, c in events]
    event_ms = (sum(fold_ms) + sum(sync_ms)) / len(events)
    # natural rate: one event per 64 steps of every instance
    ms_per_step = dec_ms / steps + event_ms / (64 * I)
    units = nl * B * (1 if p.get("joint") else H) * 2     # folded (sequence[, head], K|V)

    # ---- roofline of the decode kernel: back-to-back decode calls over the
    # layers at their current lengths, one event pair on the decode stream
    rl_calls = max(2 * nl, 64)
    rl_bytes = 0
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for c in range(rl_calls):
        layer = c % nl
        code = lib.iskv_decode_attn(ctx, layer, ctypes.c_void_p(q_base[layer % ML]), lens[layer] - 1,
                                    out_p)
        if code != 0:
            raise binding.IskvError(code, "iskv_decode_attn")
        rl_bytes += decode_bytes(p, comp[layer] - P, lens[layer] - (comp[layer] - P))
    r1.record(stream)
    torch.cuda.synchronize()
    rl_avg_ms = r0.elapsed_time(r1) / rl_calls
    bytes_avg = rl_bytes / rl_calls
    achieved = bytes_avg / (rl_avg_ms * 1e-3) / 1e9
    flags = max(cache.status(i).numeric_flags for i in range(nl))
    st = cache.status(0)
    finite = bool(torch.isfinite(out).all().item())
    res = {
        "value": B * steps / (ms_per_step * steps * 1e-3),
        "ms_per_step": ms_per_step,
        "decode_ms_per_step": dec_ms / steps,
        "instances_rotated": I,
        "layers_per_step": ML,
        "roofline": {
            "bound": "hbm", "kernel": "decode_attn", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": bytes_avg, "avg_launch_us": rl_avg_ms * 1e3,
            "launches_timed": rl_calls,
        },
        "block_updates_per_s": units * len(fold_ms) / (sum(fold_ms) * 1e-3),
        "block_updates_per_s_with_sync": units * len(fold_ms) / ((sum(fold_ms) + sum(sync_ms)) * 1e-3),
        "fold_event_units": units,
        "fold_avg_us": sum(fold_ms) / len(fold_ms) * 1e3,
        "sync_avg_us": sum(sync_ms) / len(sync_ms) * 1e3,
        "fold_events_timed": len(events),
        "step_us_max_with_fold_event": (dec_ms / steps + event_ms) * 1e3,
        "fold_events_in_steps": timed_folds,
        "prefill_s": t_pre,
        "wall_s_timed": wall,
        "numeric_flags": flags,
        "output_finite": finite,
        "persistent_kv_bytes_per_instance": st.persistent_bytes // I,
        "full_kv_bytes_per_instance": st.full_bytes // I,
        "context_at_end": max(lens),
    }
    cache.destroy()
    del cache, k_all, v_all, q_all, gen
    torch.cuda.empty_cache()
    return res


def measure_async(p, steps, warmup, instances, seed, quiet=False):
    """Copy-on-write maintenance: the same decode steps with every layer's fold
    + sync enqueued on a second stream (iskv_maintain) as soon as its block is
    ready, and switched to at a later decode boundary when finished
    (iskv_switch before each decode call; an append that would overflow the
    ring waits for it).  Timed as one interval on the decode stream, from the
    first step to the switch of the last maintenance, over enough steps that
    every instance passes three maintenances."""
    import torch

    from rank_decode_attention_iskv_amd import binding
    torch.cuda.set_device(0)
    L0, W, P, ML = p["context"], p["window"], p["prefix"], p["layers"]
    n_c0 = max(P, (L0 - W - P) // 64 * 64 + P)
    if instances <= 0:
        instances = max(1, math.ceil(ROTATE_BYTES / max(1, state_bytes(p, n_c0 - P, L0 - n_c0))))
    I = min(instances, 64)
    nl = I * ML
    steps = max(steps, 3 * 64 * I)
    per_inst = (warmup + 2 * steps + I - 1) // I
    max_tokens = L0 + per_inst + 64 * 4 + 64
    cfg = binding.make_config(p["batch"], nl, p["kv"], p["q"], 128, p["rank"], W, max_tokens,
                              p["storage"], protected_prefix=P, rank_v=p["rank_v"],
                              async_maintenance=1)
    cache = binding.IskvCache(cfg)
    ms = torch.cuda.Stream()
    cache.set_maintenance_stream(ms)
    stream = torch.cuda.current_stream()
    gen = Generator(torch, p, nl, seed)
    lib = binding.lib()
    ctx = cache.ctx

    def fold_now():
        cache.maintain(-1)
        for layer in range(nl):
            cache.switch(layer, wait=True)

    t_pre = time.perf_counter()
    length, n_c = 0, P
    while length < L0:
        n = min(256, L0 - length, W + 64 - (length - n_c) if length >= P else P - length)
        ready = False
        for layer in range(nl):
            k, v = gen.tokens(layer, n)
            ready = cache.append(layer, k, v)
        length += n
        if ready:
            fold_now()
            n_c += 64
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t_pre

    B, H, HQ = p["batch"], p["kv"], p["q"]
    tok_bytes = B * H * 128 * 4
    need = per_inst + 64 * 4
    k_all, v_all = [], []
    for layer in range(nl):
        k, v = gen.tokens(layer, need)
        k_all.append(k.permute(1, 0, 2, 3).contiguous())
        v_all.append(v.permute(1, 0, 2, 3).contiguous())
    q_all = [gen.queries(per_inst, layer) for layer in range(ML)]
    q_bytes = B * HQ * 128 * 4
    out = torch.empty(B, HQ, 128, device="cuda")
    torch.cuda.synchronize()
    k_base = [t.data_ptr() for t in k_all]
    v_base = [t.data_ptr() for t in v_all]
    q_base = [t.data_ptr() for t in q_all]
    out_p = ctypes.c_void_p(out.data_ptr())
    ready_c = ctypes.c_int(0)
    lens = [length] * nl
    used = [0] * nl
    count = {"maint": 0}

    def step(s):
        # the decode call switches a layer whose maintenance has finished
        inst = s % I
        for l in range(ML):
            layer = inst * ML + l
            j = used[layer]
            used[layer] += 1
            lens[layer] += 1
            code = lib.iskv_append_decode(ctx, layer, ctypes.c_void_p(k_base[layer] + j * tok_bytes),
                                          ctypes.c_void_p(v_base[layer] + j * tok_bytes), binding.F32,
                                          ctypes.c_void_p(q_base[l] + (s // I) * q_bytes),
                                          lens[layer] - 1, out_p, ctypes.byref(ready_c))
            if code != 0:
                raise binding.IskvError(code, "iskv_append_decode")
            if ready_c.value:
                code = lib.iskv_maintain(ctx, layer)
                if code != 0:
                    raise binding.IskvError(code, "iskv_maintain")
                count["maint"] += 1

    def run(first, n, marks=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i, s in enumerate(range(first, first + n)):
            step(s)
            if marks is not None:
                marks[i].record(stream)
        for layer in range(nl):
            cache.switch(layer, wait=True)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0, e1

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    count["maint"] = 0
    # throughput: the steps alone, then the last maintenances' switches
    e0, e1 = run(warmup, steps)
    total_ms = e0.elapsed_time(e1)
    maint_timed = count["maint"]
    # inter-token latency: the next steps again with an event after each
    n_lat = min(steps, 64 * I * 2)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_lat)]
    l0, _ = run(warmup + steps, n_lat, marks)
    gaps = sorted([l0.elapsed_time(marks[0])] + [a.elapsed_time(b) for a, b in zip(marks, marks[1:])])

    # maintenance events alone (decode stream idle): rings topped up to a
    # ready block, every layer maintained and switched, timed on the decode stream
    ev_ms = []
    for _ in range(2):
        for layer in range(nl):
            n_c_l = cache.status(layer).compressed + P
            room = W + 64 - (lens[layer] - n_c_l)
            if room > 0:
                j = used[layer]
                kk = k_all[layer][j: j + room].permute(1, 0, 2, 3).contiguous()
                vv = v_all[layer][j: j + room].permute(1, 0, 2, 3).contiguous()
                used[layer] += room
                lens[layer] += room
                cache.append(layer, kk, vv)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        fold_now()
        f1.record(stream)
        torch.cuda.synchronize()
        ev_ms.append(f0.elapsed_time(f1))
    units = nl * B * (1 if p.get("joint") else H) * 2     # folded (sequence[, head], K|V)
    flags = max(cache.status(i).numeric_flags for i in range(nl))
    finite = bool(torch.isfinite(out).all().item())
    res = {
        "value": B * steps / (total_ms * 1e-3),
        "ms_per_step": total_ms / steps,
        "steps_timed": steps,
        "instances_rotated": I,
        "maintenances_in_timed_steps": maint_timed,
        "latency_steps": n_lat,
        "maintenance_event_avg_us": sum(ev_ms) / len(ev_ms) * 1e3,
        "step_us_p50": gaps[len(gaps) // 2] * 1e3,
        "step_us_p99": gaps[min(len(gaps) - 1, (len(gaps) * 99) // 100)] * 1e3,
        "step_us_max": gaps[-1] * 1e3,
        "block_updates_per_s_with_sync": units * len(ev_ms) / (sum(ev_ms) * 1e-3),
        "prefill_s": t_pre,
        "numeric_flags": flags,
        "output_finite": finite,
    }
    cache.destroy()
    del cache, k_all, v_all, q_all, gen
    torch.cuda.empty_cache()
    return res


def prefill_compare(p, layers=16, tokens=32768, seed=77):
    """A prompt of `tokens` tokens into `layers` layers of one workload (the
    32K GQA layer: 16 instances), twice: block by block (appends of up to 64
    tokens, iskv_block_update(-1) + iskv_sync(-1) whenever the rings fill)
    and with iskv_prefill_layers (every block folded in one pass, one
    deferred synchronization per pass).  Inputs resident before timing; each
    path timed by one HIP event pair on the stream."""
    import torch

    from rank_decode_attention_iskv_amd import binding
    torch.cuda.set_device(0)
    W = p["window"]
    gen = Generator(torch, p, layers, seed)
    ks, vs = [], []
    for layer in range(layers):
        k, v = gen.tokens(layer, tokens)
        ks.append(k.contiguous())
        vs.append(v.contiguous())
    out = {"tokens": tokens, "layers": layers, "folds_per_layer": (tokens - W) // 64}
    for mode in ("block_by_block", "bulk"):
        cfg = binding.make_config(p["batch"], layers, p["kv"], p["q"], 128, p["rank"], W, tokens + 64,
                                  p["storage"], rank_v=p["rank_v"])
        cache = binding.IskvCache(cfg)
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if mode == "bulk":
            cache.prefill_layers(list(range(layers)), ks, vs)
        else:
            pos, n_c = 0, 0
            while pos < tokens:
                take = min(64, tokens - pos, W + 64 - (pos - n_c))
                ready = False
                for layer in range(layers):
                    ready = cache.append(layer, ks[layer][:, pos:pos + take].contiguous(),
                                         vs[layer][:, pos:pos + take].contiguous())
                pos += take
                if ready:
                    cache.block_update(-1)
                    cache.sync(-1)
                    n_c += 64
        e1.record(stream)
        torch.cuda.synchronize()
        out[mode + "_ms"] = e0.elapsed_time(e1)
        out[mode + "_compressed"] = cache.status(0).compressed
        cache.destroy()
    out["speedup"] = out["block_by_block_ms"] / out["bulk_ms"]
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host cores, bounded sample
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, sample_units=2, decode_calls=3):
    """The oracle (numpy float64, LAPACK) builds `sample_units` (sequence, KV
    head) units of the workload to its context, folding and syncing as the
    ring fills, then runs decode calls; with BLAS on every core of the
    process affinity and on one thread.  One step of the workload = every
    unit of every layer decodes, plus its fold + sync every 64 steps
    (averaged over the build) -- scaled linearly from the sample."""
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import JointUnit, Unit

    cores = len(os.sched_getaffinity(0))
    spectrum = "power" if p["spectrum"] == "power" else "gauss"
    joint = bool(p.get("joint"))
    heads = p["kv"] if joint else 1          # KV heads per oracle unit
    if joint:
        sample_units = 1
    w = workloads.with_(workloads.WORKLOADS[p["id"]], window=p["window"], rank=p["rank"],
                        context=p["context"], batch=1, kv_heads=heads, q_heads=heads * p["q"] // p["kv"],
                        spectrum=spectrum, shared_latent=joint)
    g = heads * p["q"] // p["kv"]
    storage = "bf16" if p["storage"] == 1 else "f32"
    runs = {}
    for threads in (cores, 1):
        with threadpool_limits(limits=threads):
            fold_t, folds, dec_t, t0 = 0.0, 0, 0.0, time.perf_counter()
            for su in range(sample_units):
                if joint:
                    u = JointUnit(heads, 128, p["rank"], p["window"], p["context"] + 64, storage,
                                  r_v=p["rank_v"])
                else:
                    u = Unit(128, p["rank"], p["window"], p["context"] + 64, storage,
                             r_v=p["rank_v"])
                pos = 0
                while pos < p["context"]:
                    n = min(64, p["context"] - pos)
                    if joint:
                        kk, vv = workloads.tokens(w, 0, pos, n)
                        k, v = kk[0], vv[0]
                    else:
                        k = workloads.unit_tokens(w, 0, su, 0, 0, pos, n)
                        v = workloads.unit_tokens(w, 0, su, 0, 1, pos, n)
                    for i in range(n):
                        u.append(k[i], v[i])
                        if u.ready:
                            f0 = time.perf_counter()
                            u.fold()
                            u.sync()
                            fold_t += time.perf_counter() - f0
                            folds += 1
                    pos += n
                d0 = time.perf_counter()
                for s in range(decode_calls):
                    q = workloads.query(w, 0, s)[0]
                    u.decode(q[:g], u.length - 1, 1.0 / math.sqrt(128))
                dec_t += (time.perf_counter() - d0) / decode_calls
            build_t = time.perf_counter() - t0
        n_units = p["layers"] * p["batch"] * p["kv"] // heads
        dec_unit = dec_t / sample_units
        fold_unit = fold_t / max(folds, 1)
        step_s = n_units * (dec_unit + fold_unit / 64.0)
        runs[threads] = dict(value=p["batch"] / step_s, decode_ms_per_unit=dec_unit * 1e3,
                             fold_sync_ms_per_unit=fold_unit * 1e3, folds=folds, build_s=build_t)
    best = max(runs, key=lambda t: runs[t]["value"])
    return {
        "value": runs[best]["value"], "unit": "tokens/s", "cores": best, "kind": "oracle",
        "sample": (f"{sample_units} (sequence, {'layer' if joint else 'KV head'}) units (K and V) "
                   f"of the workload built to "
                   f"{p['context']} tokens by the float64 oracle ({runs[best]['folds']} folds + syncs), "
                   f"then {decode_calls} decode calls of {g} query heads each; one step = "
                   f"{p['layers'] * p['batch'] * p['kv'] // heads} units x (decode + fold+sync / 64); "
                   + ("measured" if p["id"] == 1 else "extrapolated linearly from the sample")),
        "cpu_model": cpu_model(),
        "by_threads": {str(t): r for t, r in runs.items()},
    }


# ---------------------------------------------------------------------------
# ragged batch (separate measurement)
# ---------------------------------------------------------------------------

def ragged_bench(args):
    """A ragged batch: sequence b holds about context * (b + 1) / B tokens."""
    import torch

    from rank_decode_attention_iskv_amd import binding
    torch.cuda.set_device(0)
    p = preset(args, 2 if not args.context else None)
    p["batch"] = args.batch if args.batch > 1 else 16
    H, HQ, D, R, W = p["kv"], p["q"], 128, p["rank"], p["window"]
    B = p["batch"]
    RV = p["rank_v"]
    ctx_len = p["context"]
    target = [max(1, ctx_len * (b + 1) // B) for b in range(B)]
    steps = args.warmup + args.steps
    cfg = binding.make_config(B, 1, H, HQ, D, R, W, ctx_len + steps + 64, binding.BF16,
                              protected_prefix=args.protected_prefix, rank_v=RV)
    cache = binding.IskvCache(cfg)
    gen = Generator(torch, p, 1, args.seed)
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
    q_all = gen.queries(steps, 0)
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
    calls = 64
    pp = dict(p, batch=1)
    rl_bytes = sum(decode_bytes(pp, n_c[b] - args.protected_prefix,
                                length[b] - (n_c[b] - args.protected_prefix)) for b in range(B))
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
        "value": B * args.steps / total_s, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_s * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": (f"one GQA layer, ragged batch of {B} sequences at lengths "
                         f"{target[0]}..{target[-1]} (spread evenly), {H} KV / {HQ} q heads, "
                         f"head_dim {D}, rank {R} (V {RV}), window {W}, bf16 storage; per step one "
                         "token per sequence (iskv_append_ragged), iskv_decode_attn_ragged, and a "
                         "fold + sync of the sequences whose ring fills; wall-clock timing"),
            "global_batch": B, "seq_len": ctx_len, "parallelism": "single GPU",
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


def compact(r, p):
    return {
        "workload": describe(p),
        "value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
        "decode_us": r["roofline"]["avg_launch_us"],
        "roofline_frac": r["roofline"]["frac"], "achieved_GBs": r["roofline"]["achieved"],
        "algorithmic_bytes_per_launch": r["roofline"]["algorithmic_bytes_per_launch"],
        "instances_rotated": r["instances_rotated"],
        "block_updates_per_s": r["block_updates_per_s"],
        "block_updates_per_s_with_sync": r["block_updates_per_s_with_sync"],
        "fold_avg_us": r["fold_avg_us"], "sync_avg_us": r["sync_avg_us"],
        "fold_event_units": r["fold_event_units"],
        "numeric_flags": r["numeric_flags"], "output_finite": r["output_finite"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); runs over several "
              "GPUs are not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.prefill:
        print(json.dumps(prefill_compare(preset(args, 2))), flush=True)
        return
    if args.ragged:
        ragged_bench(args)
        return
    p = preset(args)
    r = measure(p, args.steps, args.warmup, args.instances, args.seed)
    kh = kernel_source_hash()
    r["roofline"]["traffic"] = committed_traffic(kh, p)
    copy_gbs = stream_bandwidth()
    r["roofline"]["measured_copy_GBs"] = copy_gbs
    r["roofline"]["frac_of_measured_copy"] = r["roofline"]["achieved"] / copy_gbs
    res = {
        "metric": METRIC,
        "value": r.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p["storage"] == 1 else "f32",
        "data": "synthetic",
        "config": {
            "workload": describe(p),
            "config_id": p["id"], "global_batch": p["batch"], "seq_len": p["context"],
            "layers": p["layers"], "rank": p["rank"], "rank_v": p["rank_v"], "window": p["window"],
            "protected_prefix": p["prefix"], "joint_heads": p["joint"], "parallelism": "single GPU",
            "step_calls": ("per layer iskv_append_decode; when the rings fill, iskv_block_update(-1) "
                           "+ iskv_sync(-1) over every layer of every instance"),
            "timing": ("decode steps timed in segments by HIP events; each fold event (block update "
                       "+ sync) timed by its own events, at least two per run; ms_per_step = decode "
                       "per step + fold event / (64 x instances), the natural rate"),
        },
    }
    res["roofline"] = r.pop("roofline")
    res.update(r)
    res["kernel_sources_sha256_16"] = kh
    if args.async_maintenance:
        a = measure_async(p, args.steps, args.warmup, args.instances, args.seed)
        res["same_stream"] = {"value": res["value"], "ms_per_step": res["ms_per_step"]}
        res["value"], res["ms_per_step"] = a.pop("value"), a.pop("ms_per_step")
        res["steps"] = a["steps_timed"]
        res["config"]["step_calls"] = (
            "per layer iskv_switch (non-blocking) + iskv_append_decode; a layer whose block is "
            "ready gets iskv_maintain (fold + sync into its other generation on a second stream)")
        res["config"]["timing"] = (
            "one HIP event interval on the decode stream over every step and the final switches; "
            "decode and maintenance overlap")
        res["async_maintenance"] = a
    if p["id"] == 3 and not args.no_extras and not (args.context or args.rank or args.window or args.batch):
        extras = {}
        p2 = preset(args, 2)
        extras["config2"] = compact(measure(p2, 128, 16, 0, args.seed + 2, quiet=True), p2)
        a2 = measure_async(p2, 128, 16, 0, args.seed + 2, quiet=True)
        extras["config2_async_maintenance"] = {
            "value": a2["value"], "unit": "tokens/s", "ms_per_step": a2["ms_per_step"],
            "same_stream_ms_per_step": extras["config2"]["ms_per_step"],
            "steps_timed": a2["steps_timed"], "maintenances": a2["maintenances_in_timed_steps"],
            "maintenance_event_avg_us": a2["maintenance_event_avg_us"],
            "step_us_p50": a2["step_us_p50"], "step_us_p99": a2["step_us_p99"],
            "step_us_max": a2["step_us_max"],
        }
        pts = []
        for rank, window in SWEEP5:
            p5 = preset(args, 5, rank=rank, rank_v=rank, window=window)
            pts.append(dict(rank=rank, window=window, **compact(measure(p5, 32, 8, 0, args.seed + 5,
                                                                        quiet=True), p5)))
        extras["config5_sweep"] = pts
        extras["config2_prefill_32k_16_layers"] = prefill_compare(preset(args, 2))
        for cid in (2, 3):
            pj = preset(args, cid, rank=64, rank_v=64, joint=1)
            extras[f"config{cid}_joint_heads_r64"] = compact(
                measure(pj, 128, 16, 0, args.seed + 10 + cid, quiet=True), pj)
        res["extras"] = extras
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(p)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
