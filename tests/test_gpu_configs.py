"""Parity at the stated sizes of the five workloads (GPU vs the float64 oracle).

  * 4,096 past tokens, 1 head, r = 32, window 256, fp32: end to end (GPU folds
    and syncs), the lone query at position 4,096;
  * 36 layers x 8 KV / 32 query heads, r = 32, window 1,024, bf16: decode at a
    65,536-token context with query positions above 32K (RoPE at 64K), and one
    block update + sync over all 36 layers in one call (576 fold workgroups);
  * batch 64 x 8K, 8 KV / 32 query heads, every (r, window) of the sweep
    (r in 16, 32, 64, 128; window 128 or 1024): decode on an imported state,
    outputs sampled per unit;
  * batch 64, 8 KV heads: one block update + sync over all 512 units (1,024
    cores, more fold workgroups than the chip holds at once), sampled units
    against the oracle;
  * the 32K GQA layer: one block update + sync on a full-size state (the sync
    rewrites all 32K old rows);
  * block update + sync on a second stream, checked against the oracle.

Full-size states are random valid states (orthonormal bases, coefficient and
ring rows) built by workloads.synthetic_unit and imported; at full size the
oracle recomputes a sample of (sequence, KV head) units one by one.
"""

import math

import numpy as np
import pytest

import workloads
from oracle import Unit
from tests.gpu_util import Pair, q32, rel_err_per_head, small, subspace_dist

pytestmark = pytest.mark.gpu

ATOL_OUT = 2e-3
HIST_BF16 = 1e-3          # rebuilt history after <= 2 folds on identical input


def _import_synthetic(w, length, n_c, max_tokens, rank_v=0, ring_in_span=False, layers=1):
    from rank_decode_attention_iskv_amd import binding
    storage = binding.BF16 if w.storage == "bf16" else binding.F32
    cfg = binding.make_config(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim, w.rank,
                              w.window, max_tokens, storage, rank_v=rank_v)
    gpu = binding.IskvCache(cfg)
    gen = (workloads.synthetic_unit(w, b, h, length, n_c, max_tokens, rank_v=rank_v,
                                    ring_in_span=ring_in_span)
           for b in range(w.batch) for h in range(w.kv_heads))
    gpu.import_state(0, binding.pack_state(cfg, length, n_c, gen))
    st = gpu.status(0)
    assert (st.length, st.compressed) == (length, n_c)
    return cfg, gpu


def _oracle_unit(w, xs, length, n_c, max_tokens, rank_v=0):
    xk, xv = xs
    u = Unit(w.head_dim, w.rank, w.window, max_tokens, w.storage, r_v=rank_v or None)
    u.load_state(length, n_c, xk["ring"], xv["ring"], xk["basis"], xk["S"], xk["coef"],
                 xv["basis"], xv["S"], xv["coef"])
    return u


def _decode(gpu, q, q_pos):
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    out = torch.empty_like(qt)
    gpu.decode_attn(0, qt, q_pos, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _sampled_decode_error(w, gpu, length, n_c, max_tokens, q_positions, units, rank_v=0):
    """max relative error over the query heads of the sampled units."""
    g = w.q_heads // w.kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    errs = []
    for step, q_pos in enumerate(q_positions):
        q = q32(workloads.query(w, 0, step))
        got = _decode(gpu, q, q_pos)
        for (b, h) in units:
            xs = workloads.synthetic_unit(w, b, h, length, n_c, max_tokens, rank_v=rank_v)
            ref = _oracle_unit(w, xs, length, n_c, max_tokens, rank_v).decode(
                q[b, h * g:(h + 1) * g], q_pos, scale)
            errs.append(rel_err_per_head(got[b, h * g:(h + 1) * g], ref))
    return max(errs)


def test_config1_end_to_end_stated_shape():
    """4,096 past tokens (3,840 compressed + 256 exact), fp32, rank-24 signal +
    1% noise: GPU appends, folds and syncs against the oracle; the lone query
    at position 4,096 (and one at 4,095)."""
    w = workloads.WORKLOADS[1]
    p = Pair(w, max_tokens=4096 + 128)
    p.feed(0, 4096)
    length, n_c, units = p.state(0)
    ora = p.ora.unit(0, 0, 0)
    assert (length, n_c) == (ora.length, ora.compressed) == (4096, 3840)
    for x, f in enumerate((ora.K, ora.V)):
        B = units[0][x]["basis"].astype(np.float64)
        assert np.linalg.norm(B.T @ B - np.eye(32), 2) < 1e-5
        assert subspace_dist(B[:, :24], f.B[:, :24]) < 1e-4      # the 24 gapped directions
        H_gpu = units[0][x]["coef"][:n_c].astype(np.float64) @ B.T
        H_ora = f.C[:n_c] @ f.B.T
        assert np.linalg.norm(H_gpu - H_ora) / np.linalg.norm(H_ora) < 1e-4
    for step, q_pos in enumerate([4096, 4095]):
        q = q32(workloads.query(w, 0, step))
        err = rel_err_per_head(p.decode(0, q, q_pos), p.ora.decode_attn(0, q, q_pos))
        assert err < ATOL_OUT, (q_pos, err)


def test_config4_decode_at_64k_context():
    """One layer of the 36-layer model at its final size: 65,536 tokens
    (64,512 compressed + 1,024 exact), window 1,024, r = 32, 8 KV / 32 query
    heads (queries with the hot direction), bf16; every query head checked at
    positions above 32K."""
    w = workloads.with_(workloads.WORKLOADS[4], num_layers=1)
    length, n_c = 65536, 64512
    max_tokens = length + 64
    cfg, gpu = _import_synthetic(w, length, n_c, max_tokens)
    units = [(0, h) for h in range(w.kv_heads)]
    err = _sampled_decode_error(w, gpu, length, n_c, max_tokens,
                                [65535, 32769, 49999, 65536 + 40], units)
    gpu.destroy()
    assert err < ATOL_OUT, err


def test_config4_all_36_layers_block_update_and_sync():
    """36 layers x 8 KV heads, window 1,024, r = 32, bf16, hot keys: every
    layer filled to a full ring, then iskv_block_update(-1) + iskv_sync(-1)
    twice (576 fold workgroups per call on 256 CUs; the second sync rewrites
    the first block).  Every layer's history and three layers' outputs against
    the oracle fed the same stream."""
    w = workloads.WORKLOADS[4]
    layers = w.num_layers
    L1 = w.window + 64
    p = Pair(w, max_tokens=L1 + 192, layers=layers)
    import torch
    for rnd, n in enumerate((L1, 64)):
        for layer in range(layers):
            k, v = workloads.tokens(w, layer, p.length[layer], n)
            k32, v32 = k.astype(np.float32), v.astype(np.float32)
            ready = p.gpu.append(layer, torch.from_numpy(k32).cuda(), torch.from_numpy(v32).cuda())
            assert ready
            p.ora.append(layer, k32.astype(np.float64), v32.astype(np.float64))
            p.length[layer] += n
        p.gpu.block_update(-1)
        p.gpu.sync(-1)
        for layer in range(layers):
            p.ora.block_update(layer)
            p.ora.sync(layer)
    worst = 0.0
    for layer in range(layers):
        length, n_c, units = p.state(layer)
        assert (length, n_c) == (L1 + 64, 128)
        for h in range(w.kv_heads):
            ou = p.ora.unit(0, layer, h)
            for x, f in enumerate((ou.K, ou.V)):
                Hg = units[h][x]["coef"][:n_c].astype(np.float64) @ units[h][x]["basis"].T
                Ho = f.C[:n_c] @ f.B.T
                worst = max(worst, float(np.linalg.norm(Hg - Ho) / np.linalg.norm(Ho)))
    assert worst < HIST_BF16, worst
    for layer in (0, 17, 35):
        q = q32(workloads.query(w, layer, 0))
        err = rel_err_per_head(p.decode(layer, q, L1 + 63), p.ora.decode_attn(layer, q, L1 + 63))
        assert err < ATOL_OUT, (layer, err)


@pytest.mark.parametrize("rank,window", [(r, w) for r in (16, 32, 64, 128) for w in (128, 1024)])
def test_config5_batch64_8k_decode(rank, window):
    """Batch 64 x 8,192 tokens, 8 KV / 32 query heads, bf16, at every point of
    the sweep (r x window); every unit's output is computed on the GPU, twelve sampled
    (sequence, KV head) units are recomputed by the oracle."""
    w = workloads.with_(workloads.WORKLOADS[5], rank=rank, window=window)
    length = 8192
    n_c = length - window
    max_tokens = length + 64
    cfg, gpu = _import_synthetic(w, length, n_c, max_tokens)
    units = [(0, 0), (0, 7), (1, 3), (13, 5), (31, 1), (32, 6), (40, 2), (47, 4), (55, 0),
             (62, 7), (63, 0), (63, 7)]
    err = _sampled_decode_error(w, gpu, length, n_c, max_tokens, [length - 1], units)
    gpu.destroy()
    assert err < ATOL_OUT, err



@pytest.mark.parametrize("rank,window", [(32, 128), (128, 1024)])
def test_config5_batch64_fold_and_sync(rank, window):
    """Batch 64, 8 KV / 32 query heads, bf16, a full ring in every unit: one
    block update + sync folds 64 x 8 x 2 = 1,024 cores of size (r + 64)^2 in
    one call; the rebuilt histories and the decode of sampled units are
    compared with the oracle's fold + sync of the same imported state."""
    w = workloads.with_(workloads.WORKLOADS[5], rank=rank, window=window)
    n_c = 1024
    length = n_c + window + 64
    max_tokens = length + 64
    cfg, gpu = _import_synthetic(w, length, n_c, max_tokens, ring_in_span=True)
    assert gpu.status(0).blocks_ready == 1
    gpu.block_update(0)
    gpu.sync(0)
    from rank_decode_attention_iskv_amd import binding
    _, n_c2, got = binding.unpack_state(cfg, gpu.export_state(0))
    assert n_c2 == n_c + 64
    units = [(0, 0), (1, 3), (13, 5), (31, 1), (47, 4), (63, 7)]
    g = w.q_heads // w.kv_heads
    q = q32(workloads.query(w, 0, 0))
    out = _decode(gpu, q, length - 1)
    gpu.destroy()
    worst_hist = worst_out = 0.0
    for (b, h) in units:
        u = _oracle_unit(w, workloads.synthetic_unit(w, b, h, length, n_c, max_tokens,
                                                     ring_in_span=True), length, n_c, max_tokens)
        u.fold()
        u.sync()
        for x, f in enumerate((u.K, u.V)):
            gu = got[b * w.kv_heads + h][x]
            Hg = gu["coef"][:n_c2].astype(np.float64) @ gu["basis"].T
            Ho = f.C[:n_c2] @ f.B.T
            worst_hist = max(worst_hist, float(np.linalg.norm(Hg - Ho) / np.linalg.norm(Ho)))
        ref = u.decode(q[b, h * g:(h + 1) * g], length - 1, 1.0 / math.sqrt(w.head_dim))
        worst_out = max(worst_out, rel_err_per_head(out[b, h * g:(h + 1) * g], ref))
    print(f"batch-64 fold r={rank} W={window}: history {worst_hist:.2e}, decode {worst_out:.2e}")
    assert worst_hist < HIST_BF16, worst_hist
    assert worst_out < ATOL_OUT, worst_out


def test_config2_fold_and_sync_at_full_history():
    """The 32K GQA layer (8 KV / 32 query heads, r = 32, window 256, bf16) with
    a full ring: one block update + sync on the imported state rewrites all
    32,448 old coefficient rows; GPU vs oracle on every unit."""
    w = workloads.WORKLOADS[2]
    n_c = 32448
    length = n_c + w.window + 64
    max_tokens = length + 64
    cfg, gpu = _import_synthetic(w, length, n_c, max_tokens, ring_in_span=True)
    assert gpu.status(0).blocks_ready == 1
    gpu.block_update(0)
    gpu.sync(0)
    from rank_decode_attention_iskv_amd import binding
    _, n_c2, got = binding.unpack_state(cfg, gpu.export_state(0))
    assert n_c2 == n_c + 64
    oras = []
    worst = 0.0
    for h in range(w.kv_heads):
        u = _oracle_unit(w, workloads.synthetic_unit(w, 0, h, length, n_c, max_tokens,
                                                     ring_in_span=True), length, n_c, max_tokens)
        u.fold()
        u.sync()
        oras.append(u)
        for x, f in enumerate((u.K, u.V)):
            Hg = got[h][x]["coef"][:n_c2].astype(np.float64) @ got[h][x]["basis"].T
            Ho = f.C[:n_c2] @ f.B.T
            worst = max(worst, float(np.linalg.norm(Hg - Ho) / np.linalg.norm(Ho)))
    assert worst < HIST_BF16, worst
    g = w.q_heads // w.kv_heads
    q = q32(workloads.query(w, 0, 0))
    out = _decode(gpu, q, length - 1)
    gpu.destroy()
    for h, u in enumerate(oras):
        ref = u.decode(q[0, h * g:(h + 1) * g], length - 1, 1.0 / math.sqrt(w.head_dim))
        assert rel_err_per_head(out[0, h * g:(h + 1) * g], ref) < ATOL_OUT


def test_maintenance_stream_matches_oracle():
    """Block updates and syncs on a second stream (fp32 storage, two layers
    interleaved): every decode matches the oracle fed the same stream."""
    import torch
    w = small(1, kv_heads=2, q_heads=4, window=128)
    p = Pair(w, max_tokens=64 * 14 + 256, layers=2)
    p.gpu.set_maintenance_stream(torch.cuda.Stream())
    for rnd in range(10):
        for layer in (0, 1):
            p.feed(layer, 64 + 5 * layer)
            q = q32(workloads.query(w, layer, rnd))
            L = p.length[layer]
            err = rel_err_per_head(p.decode(layer, q, L - 1), p.ora.decode_attn(layer, q, L - 1))
            assert err < ATOL_OUT, (rnd, layer, err)
    p.gpu.join_maintenance()
    assert p.gpu.status(0).folds >= 8
