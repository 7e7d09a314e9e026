"""Ragged batches: the sequences of one batch at their own lengths and fold
steps (iskv_append_ragged, iskv_decode_attn_ragged, per-sequence folds).

Not on the pages (a serving need: every sequence is its own stream).  Each
sequence's state must be the one a single-sequence cache fed the same stream
reaches, so the checks are: the oracle run per sequence (f32, end to end),
one batch-1 cache per sequence (bf16: the fold kernels see the same unit data,
so only the decode's split boundaries differ), and bit-identity with the
uniform calls when every sequence advances together.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import Oracle
from tests.gpu_util import q32, rel_err_per_head, small

pytestmark = pytest.mark.gpu

ATOL_OUT = 2e-3


def seq_tokens(w, b, start, n):
    """Sequence b's tokens start..start+n-1 as [n, kv_heads, d] (K, V)."""
    k = np.stack([workloads.unit_tokens(w, b, 0, h, 0, start, n) for h in range(w.kv_heads)], axis=1)
    v = np.stack([workloads.unit_tokens(w, b, 0, h, 1, start, n) for h in range(w.kv_heads)], axis=1)
    return k.astype(np.float32), v.astype(np.float32)


class Ragged:
    """A GPU cache driven with ragged appends, and the oracle fed per sequence."""

    def __init__(self, w, max_tokens, prefix=0, oracle=True):
        import torch
        from rank_decode_attention_iskv_amd import binding
        self.torch, self.binding, self.w = torch, binding, w
        storage = binding.BF16 if w.storage == "bf16" else binding.F32
        self.cfg = binding.make_config(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank,
                                       w.window, max_tokens, storage, protected_prefix=prefix)
        self.gpu = binding.IskvCache(self.cfg)
        self.ora = (Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                           max_tokens, storage=w.storage, prefix=prefix) if oracle else None)
        self.prefix = prefix
        self.length = [0] * w.batch
        self.n_c = [prefix] * w.batch
        self.folds = [0] * w.batch

    def free(self, b):
        """Tokens sequence b can take before its ring is full."""
        slots = self.w.window + 64
        return slots - (self.length[b] - self.n_c[b]) if self.length[b] >= self.prefix else \
            self.prefix - self.length[b] + slots

    def step(self, counts):
        torch, w = self.torch, self.w
        n = max(max(counts), 1)
        K = np.zeros((w.batch, n, w.kv_heads, w.head_dim), np.float32)
        V = np.zeros_like(K)
        for b, c in enumerate(counts):
            if c:
                K[b, :c], V[b, :c] = seq_tokens(w, b, self.length[b], c)
        ready = self.gpu.append_ragged(0, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(),
                                       counts)
        for b, c in enumerate(counts):
            if self.ora is not None:
                for t in range(c):
                    for h in range(w.kv_heads):
                        self.ora.unit(b, 0, h).append(K[b, t, h].astype(np.float64),
                                                      V[b, t, h].astype(np.float64))
            self.length[b] += c
        full = [b for b in range(w.batch) if self.length[b] - self.n_c[b] == w.window + 64]
        assert ready == len(full)
        if full:
            self.gpu.block_update(0)
            self.gpu.sync(0)
            for b in full:
                self.n_c[b] += 64
                self.folds[b] += 1
                if self.ora is not None:
                    for h in range(w.kv_heads):
                        u = self.ora.unit(b, 0, h)
                        assert u.ready
                        u.fold()
                        u.sync()
        return full

    def decode(self, q, q_pos):
        torch = self.torch
        qt = torch.from_numpy(np.asarray(q, np.float32)).cuda()
        out = torch.empty_like(qt)
        self.gpu.decode_attn_ragged(0, qt, q_pos, out)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    def oracle_decode(self, q, q_pos):
        w = self.w
        g = w.q_heads // w.kv_heads
        out = np.zeros((w.batch, w.q_heads, w.head_dim))
        for b in range(w.batch):
            for h in range(w.kv_heads):
                out[b, h * g:(h + 1) * g] = self.ora.unit(b, 0, h).decode(
                    q[b, h * g:(h + 1) * g], q_pos[b], 1.0 / math.sqrt(w.head_dim))
        return out


def schedule(rng, r, limit):
    """Seeded per-sequence counts: bursts, single tokens and pauses."""
    counts = []
    for b in range(r.w.batch):
        c = int(rng.choice([0, 1, 1, 3, 17, 40, 64]))
        counts.append(min(c, r.free(b), limit - r.length[b]))
    return counts


@pytest.mark.parametrize("wid,kw,prefix", [
    (1, dict(batch=3, kv_heads=2, q_heads=4, window=128), 0),              # f32 r=32
    (1, dict(batch=4, kv_heads=1, q_heads=4, window=64, rank=16), 128),     # f32 r=16, prefix
])
def test_ragged_end_to_end_f32(wid, kw, prefix):
    """Per-sequence appends of different sizes, folds at different steps, and
    decode at per-sequence positions against the oracle run per sequence."""
    w = small(wid, **kw)
    limit = 1100
    r = Ragged(w, limit + 64, prefix=prefix)
    rng = np.random.default_rng(70 + w.rank)
    checks = 0
    for step in range(60):
        r.step(schedule(rng, r, limit))
        if step % 6 == 5 and min(r.length) > 0:
            q = q32(workloads.query(w, 0, step))
            q_pos = [L - 1 + 3 * (b % 2) for b, L in enumerate(r.length)]
            got = r.decode(q, q_pos)
            ref = r.oracle_decode(q, q_pos)
            assert rel_err_per_head(got, ref) < ATOL_OUT, (step, rel_err_per_head(got, ref))
            checks += 1
    for b in range(w.batch):
        st = r.gpu.seq_status(0, b)
        u = r.ora.unit(b, 0, 0)
        assert (st.length, st.compressed) == (u.length, u.compressed)
    assert checks >= 5
    assert len(set(r.length)) > 1 and len(set(r.folds)) > 1   # really ragged
    assert max(r.folds) >= 3


def test_ragged_bf16_matches_single_sequence_caches():
    """bf16, G=4, r=32: a batch of 3 ragged sequences against three batch-1
    caches fed the same streams with the uniform calls.  Folds and syncs see
    the same unit data, so every output agrees up to the decode's split
    boundaries (fp32 summation order)."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = small(2, batch=3, kv_heads=2, q_heads=8, window=128)
    limit = 1500
    r = Ragged(w, limit + 64, oracle=False)
    singles = []
    for b in range(w.batch):
        cfg = binding.make_config(1, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                                  limit + 64, binding.BF16)
        singles.append(binding.IskvCache(cfg))
    rng = np.random.default_rng(81)
    checks = 0
    for step in range(70):
        start = list(r.length)
        counts = schedule(rng, r, limit)
        full = r.step(counts)
        for b, c in enumerate(counts):
            if not c:
                continue
            k, v = seq_tokens(w, b, start[b], c)
            ready = singles[b].append(0, torch.from_numpy(k[None]).cuda(), torch.from_numpy(v[None]).cuda())
            assert ready == (b in full)
            if ready:
                singles[b].block_update(0)
                singles[b].sync(0)
        if step % 7 == 6 and min(r.length) > 0:
            q = q32(workloads.query(w, 0, step))
            q_pos = [L + 2 for L in r.length]
            got = r.decode(q, q_pos)
            for b in range(w.batch):
                qt = torch.from_numpy(q[b:b + 1].astype(np.float32)).cuda()
                out = torch.empty_like(qt)
                singles[b].decode_attn(0, qt, q_pos[b], out)
                torch.cuda.synchronize()
                ref = out.cpu().numpy().astype(np.float64)
                # different split boundaries give each side its own
                # reference max, so p = 2^(s - m) is rounded differently
                # where it is split into bf16 hi + lo for the value product
                # (~2^-17 relative per weight): agreement to a few 1e-5
                assert rel_err_per_head(got[b:b + 1], ref) < 5e-5, (step, b)
            checks += 1
    assert checks >= 5 and len(set(r.folds)) > 1 and max(r.folds) >= 4


def test_ragged_equal_counts_bit_identical_to_uniform():
    """When every sequence takes the same count the ragged calls give the same
    bits as iskv_append / iskv_decode_attn, and the layer turns uniform again
    (iskv_status, iskv_export_state work)."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = small(2, batch=2, kv_heads=2, q_heads=8, window=64)
    limit = 700
    a = Ragged(w, limit + 64, oracle=False)
    cfg = binding.make_config(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              limit + 64, binding.BF16)
    u = binding.IskvCache(cfg)
    pos = 0
    for step, n in enumerate([40, 24, 64, 1, 63, 64, 7, 57, 64, 64, 30]):
        n = min(n, a.free(0))
        start = pos
        a.step([n] * w.batch)
        k, v = workloads.tokens(w, 0, start, n)
        ready = u.append(0, torch.from_numpy(k.astype(np.float32)).cuda(),
                         torch.from_numpy(v.astype(np.float32)).cuda())
        pos += n
        if ready:
            u.block_update(0)
            u.sync(0)
        q = q32(workloads.query(w, 0, step))
        got = a.decode(q, [pos - 1] * w.batch)
        qt = torch.from_numpy(q.astype(np.float32)).cuda()
        out = torch.empty_like(qt)
        u.decode_attn(0, qt, pos - 1, out)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, out.cpu().numpy().astype(np.float64))
    assert a.gpu.status(0).length == pos == u.status(0).length
    assert bytes(a.gpu.export_state(0)) == bytes(u.export_state(0))


def test_ragged_uniform_calls_refuse_differing_sequences():
    from rank_decode_attention_iskv_amd import binding
    w = small(2, batch=2, kv_heads=1, q_heads=4, window=64)
    r = Ragged(w, 512, oracle=False)
    r.step([5, 9])
    with pytest.raises(binding.IskvError):
        r.gpu.status(0)
    with pytest.raises(binding.IskvError):
        r.gpu.export_state(0)
    assert [r.gpu.seq_status(0, b).length for b in range(2)] == [5, 9]
    r.step([4, 0])                                 # equal again: uniform calls work
    assert r.gpu.status(0).length == 9


def test_ragged_and_uniform_layers_fold_together():
    """iskv_block_update(-1) / iskv_sync(-1) over a ragged layer and a uniform
    layer give the same bits as the per-layer calls."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = small(2, batch=3, kv_heads=2, q_heads=8, window=64)
    cfg = binding.make_config(w.batch, 2, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              1024, binding.BF16)
    caches = [binding.IskvCache(cfg), binding.IskvCache(cfg)]
    rng = np.random.default_rng(5)
    length = [[0] * w.batch, [0] * w.batch]
    n_c = [[0] * w.batch, [0] * w.batch]
    folds = 0
    for step in range(24):
        c0 = [int(min(rng.integers(0, 50), 128 - (length[0][b] - n_c[0][b]))) for b in range(w.batch)]
        n1 = int(min(rng.integers(1, 50), 128 - (length[1][0] - n_c[1][0])))
        n = max(max(c0), 1)
        K0 = np.zeros((w.batch, n, w.kv_heads, w.head_dim), np.float32)
        V0 = np.zeros_like(K0)
        for b, c in enumerate(c0):
            if c:
                K0[b, :c], V0[b, :c] = seq_tokens(w, b, length[0][b], c)
        k1, v1 = workloads.tokens(w, 1, length[1][0], n1)
        for ci, cache in enumerate(caches):
            cache.append_ragged(0, torch.from_numpy(K0).cuda(), torch.from_numpy(V0).cuda(), c0)
            cache.append(1, torch.from_numpy(k1.astype(np.float32)).cuda(),
                         torch.from_numpy(v1.astype(np.float32)).cuda())
        for b in range(w.batch):
            length[0][b] += c0[b]
            length[1][b] += n1
        full0 = [b for b in range(w.batch) if length[0][b] - n_c[0][b] == 128]
        full1 = length[1][0] - n_c[1][0] == 128
        if full0 or full1:
            caches[0].block_update(-1)
            caches[0].sync(-1)
            if full0:
                caches[1].block_update(0)
                caches[1].sync(0)
            if full1:
                caches[1].block_update(1)
                caches[1].sync(1)
            for b in full0:
                n_c[0][b] += 64
            if full1:
                for b in range(w.batch):
                    n_c[1][b] += 64
            folds += 1
    assert folds >= 4 and len(set(n_c[0])) > 1
    q = torch.from_numpy(q32(workloads.query(w, 0, 3)).astype(np.float32)).cuda()
    outs = []
    for cache in caches:
        o0, o1 = torch.empty_like(q), torch.empty_like(q)
        cache.decode_attn_ragged(0, q, [L + 1 for L in length[0]], o0)
        cache.decode_attn(1, q, length[1][0] - 1, o1)
        torch.cuda.synchronize()
        outs.append((o0.cpu().numpy(), o1.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    for b in range(w.batch):
        assert caches[0].seq_status(0, b).compressed == caches[1].seq_status(0, b).compressed == n_c[0][b]


def test_ragged_widely_unequal_lengths_match_single_sequence_caches():
    """bf16, G=4, r=32, window 128: 8 sequences held at 192 .. 3,072 tokens.
    For these lengths the four-wave decode plan leaves each wave fewer tokens
    than the eight-wave one (280 vs 2 x 128 tokens a workgroup), so the
    ragged call takes the four-wave form while its eight-wave grid would fit;
    every sequence's output agrees with a batch-1 cache fed the same stream."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    target = [192, 384, 640, 1024, 1536, 2048, 2560, 3072]
    w = small(2, batch=len(target), kv_heads=2, q_heads=8, window=128)
    limit = max(target)
    r = Ragged(w, limit + 64, oracle=False)
    singles = []
    for b in range(w.batch):
        cfg = binding.make_config(1, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                                  limit + 64, binding.BF16)
        singles.append(binding.IskvCache(cfg))
    while r.length != target:
        start = list(r.length)
        counts = [min(64, r.free(b), target[b] - r.length[b]) for b in range(w.batch)]
        full = r.step(counts)
        for b, c in enumerate(counts):
            if not c:
                continue
            k, v = seq_tokens(w, b, start[b], c)
            ready = singles[b].append(0, torch.from_numpy(k[None]).cuda(), torch.from_numpy(v[None]).cuda())
            assert ready == (b in full)
            if ready:
                singles[b].block_update(0)
                singles[b].sync(0)
    q = q32(workloads.query(w, 0, 5))
    q_pos = [L + 2 for L in r.length]
    got = r.decode(q, q_pos)
    errs = []
    for b in range(w.batch):
        qt = torch.from_numpy(q[b:b + 1].astype(np.float32)).cuda()
        out = torch.empty_like(qt)
        singles[b].decode_attn(0, qt, q_pos[b], out)
        torch.cuda.synchronize()
        errs.append(rel_err_per_head(got[b:b + 1], out.cpu().numpy().astype(np.float64)))
    print(f"widely unequal ragged batch vs batch-1 caches: {max(errs):.2e}")
    # split boundaries differ between the two sides (see the bound above)
    assert max(errs) < 5e-5, errs
    assert min(r.folds) >= 1 and max(r.folds) >= 40
