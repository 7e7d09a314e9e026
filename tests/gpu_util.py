"""Drive the GPU library and the float64 oracle with the same seeded stream.

The oracle only ever receives the synthetic inputs (rounded to float32, the
dtype handed to the GPU), never a value produced by the GPU.
"""

from __future__ import annotations

import math

import numpy as np

import workloads
from oracle import Oracle


def rel_err_per_head(got, ref):
    """max over (sequence, query head) of ||got - ref|| / ||ref||."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / den))


def subspace_dist(B1, B2):
    Q1, _ = np.linalg.qr(np.asarray(B1, np.float64))
    Q2, _ = np.linalg.qr(np.asarray(B2, np.float64))
    return float(np.linalg.norm(Q1 @ Q1.T - Q2 @ Q2.T, 2))


class Pair:
    """A GPU cache and an oracle fed with identical float32 inputs."""

    def __init__(self, w: workloads.Workload, max_tokens=None, oracle=True, layers=1, prefix=0,
                 rank_v=0, joint=False):
        import torch
        from rank_decode_attention_iskv_amd import binding
        self.torch, self.binding, self.w = torch, binding, w
        self.layers = layers
        self.max_tokens = max_tokens or w.context + 64
        storage = binding.BF16 if w.storage == "bf16" else binding.F32
        self.prefix = prefix
        self.cfg = binding.make_config(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim,
                                       w.rank, w.window, self.max_tokens, storage,
                                       protected_prefix=prefix, rank_v=rank_v,
                                       joint_heads=int(joint))
        self.joint = joint
        self.gpu = binding.IskvCache(self.cfg)
        self.ora = (Oracle(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                           self.max_tokens, storage=w.storage, prefix=prefix,
                           rank_v=rank_v or None, joint_heads=joint) if oracle else None)
        self.length = [0] * layers

    def feed(self, layer, count, sync=True, chunk=64, on_fold=None):
        """Append `count` tokens of the workload stream, folding (and syncing)
        whenever the ring fills."""
        torch = self.torch
        slots = self.w.window + 64
        end = self.length[layer] + count
        while self.length[layer] < end:
            st = self.gpu.status(layer)
            # ring positions start at prefix + compressed; earlier ones fill the prefix
            free = slots - (st.length - self.prefix - st.compressed)
            n = min(chunk, free, end - self.length[layer])
            k, v = workloads.tokens(self.w, layer, self.length[layer], n)
            k32, v32 = k.astype(np.float32), v.astype(np.float32)
            ready = self.gpu.append(layer, torch.from_numpy(k32).cuda(), torch.from_numpy(v32).cuda())
            if self.ora is not None:
                self.ora.append(layer, k32.astype(np.float64), v32.astype(np.float64))
            self.length[layer] += n
            if ready:
                self.gpu.block_update(layer)
                if self.ora is not None:
                    self.ora.block_update(layer)
                if sync:
                    self.gpu.sync(layer)
                    if self.ora is not None:
                        self.ora.sync(layer)
                else:
                    self.gpu.discard_sync(layer)
                    if self.ora is not None:
                        for b in range(self.w.batch):
                            for h in range(self.w.kv_heads):
                                u = self.ora.unit(b, layer, h)
                                u.K.pending = u.V.pending = None
                if on_fold:
                    on_fold(self)

    def decode(self, layer, q, q_pos):
        torch = self.torch
        qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
        out = torch.empty_like(qt)
        self.gpu.decode_attn(layer, qt, q_pos, out)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    def state(self, layer):
        return self.binding.unpack_state(self.cfg, self.gpu.export_state(layer))

    def oracle_blob(self, layer):
        """State blob made from the oracle's state (for iskv_import_state)."""
        w = self.w
        units = []
        d = w.head_dim
        for b in range(w.batch):
            for h in range(w.kv_heads):
                u = self.ora.unit(b, layer, h)
                # a joint unit's rows are its heads' rows side by side: head h
                # lists its slice of the basis, ring and prefix columns
                cols = slice(h * d, (h + 1) * d) if self.joint else slice(None)
                units.append([dict(basis=f.B[cols], S=f.S, coef=f.C[: u.n_c], ring=f.ring[:, cols],
                                   prefix=f.prefix[:, cols]) for f in (u.K, u.V)])
        u0 = self.ora.unit(0, layer, 0)
        return self.binding.pack_state(self.cfg, u0.length, u0.compressed, units)


def exact_attention(w, L, q, q_pos):
    """Uncompressed attention over the first L stream tokens, stored at the
    workload's precision (float64 result; keys rotated at their positions)."""
    from oracle import rope, store_round
    out = np.zeros((w.batch, w.q_heads, w.head_dim))
    g = w.q_heads // w.kv_heads
    k, v = workloads.tokens(w, 0, 0, L)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            kk = store_round(k[b, :, h].astype(np.float32).astype(np.float64), w.storage)
            vv = store_round(v[b, :, h].astype(np.float32).astype(np.float64), w.storage)
            qr = rope(q[b, h * g:(h + 1) * g], q_pos)
            s = qr @ rope(kk, np.arange(L)).T / math.sqrt(w.head_dim)
            pr = np.exp(s - s.max(1, keepdims=True))
            out[b, h * g:(h + 1) * g] = (pr / pr.sum(1, keepdims=True)) @ vv
    return out


def q32(q):
    """Queries as the GPU receives them (float32), in float64 for the oracle."""
    return np.asarray(q, dtype=np.float32).astype(np.float64)


def small(w_id, **kw):
    return workloads.with_(workloads.WORKLOADS[w_id], **kw)


def scale(w):
    return 1.0 / math.sqrt(w.head_dim)
