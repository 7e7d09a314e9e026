"""Bulk prefill (iskv_prefill) against the oracle and against the
block-by-block path on the GPU.

iskv_prefill folds every block of a prompt that leaves the window in one
pass, reading the blocks from the input, and synchronizes the older rows once
with the product of the later M's.  The oracle's Unit.prefill does the same
in float64 and is pinned on the CPU to block-by-block folding + sync
(test_oracle_pins).  On the GPU the folds are the same kernel code as the
block-by-block path, so with bf16 storage bases and singular values match it
bit for bit; only the older coefficient rows differ, by where the products
round.
"""

import math
import os

import numpy as np
import pytest

import workloads
from oracle import Oracle
from tests.gpu_util import q32, rel_err_per_head, small, subspace_dist

pytestmark = pytest.mark.gpu


def _cache(w, max_tokens, prefix=0, rank_v=0):
    from rank_decode_attention_iskv_amd import binding
    storage = binding.BF16 if w.storage == "bf16" else binding.F32
    cfg = binding.make_config(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              max_tokens, storage, protected_prefix=prefix, rank_v=rank_v)
    return cfg, binding.IskvCache(cfg)


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _history(cfg, gpu):
    from rank_decode_attention_iskv_amd import binding
    length, n_c, units = binding.unpack_state(cfg, gpu.export_state(0))
    P = cfg.protected_prefix
    return length, n_c, [[u[x]["coef"][P:P + n_c].astype(np.float64) @ u[x]["basis"].T.astype(np.float64)
                          for x in (0, 1)] for u in units], units


def _decode(gpu, q, q_pos):
    import torch
    qt = _dev(q)
    out = torch.empty_like(qt)
    gpu.decode_attn(0, qt, q_pos, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("bulk_blocks,prefix,rank_v", [(0, 0, 0), (3, 0, 0), (0, 64, 0), (4, 64, 64)])
def test_prefill_matches_oracle_f32(bulk_blocks, prefix, rank_v, monkeypatch):
    """fp32 storage, 2 sequences x 2 KV heads, r = 32 (V at 64 in one case):
    a prompt of window + 9 blocks + 37 tokens in one call (in passes of 3 or 4
    blocks when the M slots are limited) against the oracle's bulk prefill;
    then decoding continues block by block."""
    if bulk_blocks:
        monkeypatch.setenv("ISKV_BULK_BLOCKS", str(bulk_blocks))
    w = small(1, batch=2, kv_heads=2, q_heads=8, window=128, rank=32)
    n = 128 + 64 * 9 + 37
    cfg, gpu = _cache(w, prefix + n + 256, prefix, rank_v)
    ora = Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, prefix + n + 256,
                 storage="f32", prefix=prefix, rank_v=rank_v or None)
    k, v = workloads.tokens(w, 0, 0, prefix + n)
    k32, v32 = k.astype(np.float32), v.astype(np.float32)
    if prefix:
        gpu.append(0, _dev(k32[:, :prefix]), _dev(v32[:, :prefix]))
        ora.append(0, k32[:, :prefix].astype(np.float64), v32[:, :prefix].astype(np.float64))
    gpu.prefill(0, _dev(k32[:, prefix:]), _dev(v32[:, prefix:]))
    ora.prefill(0, k32[:, prefix:].astype(np.float64), v32[:, prefix:].astype(np.float64))
    st = gpu.status(0)
    assert (st.length, st.compressed, st.folds) == (prefix + n, 64 * 9, 9)
    length, n_c, hist, units = _history(cfg, gpu)
    worst = [0.0, 0.0]
    for b in range(w.batch):
        for h in range(w.kv_heads):
            ou = ora.unit(b, 0, h)
            for x, f in enumerate((ou.K, ou.V)):
                Ho = f.C[prefix:prefix + n_c] @ f.B.T
                worst[x] = max(worst[x], float(np.linalg.norm(hist[b * w.kv_heads + h][x] - Ho) /
                                               np.linalg.norm(Ho)))
    assert worst[0] < 1e-5, worst
    # a V rank of 64 on a rank-24 signal keeps 40 noise directions of nearly
    # equal singular values: which ones (fp32 vs fp64) moves the rebuilt
    # history by ~1e-3 of its norm, in every block alike (the fold, not the
    # deferred synchronization); the outputs below stay at ~1e-5
    assert worst[1] < (2e-3 if rank_v > w.signal_rank else 1e-5), worst
    errs = []
    for step in range(3):
        q = q32(workloads.query(w, 0, step))
        errs.append(rel_err_per_head(_decode(gpu, q, prefix + n - 1 - step), ora.decode_attn(0, q, prefix + n - 1 - step)))
    # decoding continues: 100 more tokens, folding block by block
    k2, v2 = workloads.tokens(w, 0, prefix + n, 100)
    for t in range(100):
        kk, vv = k2[:, t:t + 1].astype(np.float32), v2[:, t:t + 1].astype(np.float32)
        ready = gpu.append(0, _dev(kk), _dev(vv))
        ora.append(0, kk.astype(np.float64), vv.astype(np.float64))
        if ready:
            gpu.block_update(0)
            gpu.sync(0)
            ora.block_update(0)
            ora.sync(0)
    q = q32(workloads.query(w, 0, 9))
    errs.append(rel_err_per_head(_decode(gpu, q, prefix + n + 99), ora.decode_attn(0, q, prefix + n + 99)))
    gpu.destroy()
    print(f"prefill f32: history K {worst[0]:.2e} V {worst[1]:.2e}, outputs {max(errs):.2e}")
    assert max(errs) < 2e-3, errs


def test_prefill_bf16_against_oracle_and_block_by_block():
    """bf16 storage, 8 KV / 32 query heads, r = 32, a 2,048-token prompt
    (28 folds): bases and singular values bit-identical to appending +
    folding + syncing block by block on the GPU (the same fold code on the
    same rounded rows); the history and the decode outputs against the
    oracle's bulk prefill in bf16 (rows rounded where the GPU rounds them: the
    block's own coefficients, then once after the deferred synchronization).
    Block by block, the oldest rows are re-rounded at every sync (20 times
    here) and drift from the single-rounding result by several bf16 ulps --
    reported, not gated.  Against the oracle, 20 folds in bf16 are an
    end-to-end run: its outputs are bounded by the bf16 walk envelope at 20
    folds (tests/test_oracle_bf16_walk.py), the history by 2e-3."""
    from tests.test_oracle_bf16_walk import WALK_ENVELOPE
    w = small(2, window=256)
    n = 256 + 64 * 20
    k, v = workloads.tokens(w, 0, 0, n)
    k32, v32 = k.astype(np.float32), v.astype(np.float32)
    cfg_a, a = _cache(w, n + 64)
    a.prefill(0, _dev(k32), _dev(v32))
    cfg_b, b = _cache(w, n + 64)
    pos = 0
    while pos < n:
        st = b.status(0)
        take = min(64, n - pos, w.window + 64 - (st.length - st.compressed))
        if b.append(0, _dev(k32[:, pos:pos + take]), _dev(v32[:, pos:pos + take])):
            b.block_update(0)
            b.sync(0)
        pos += take
    ora = Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, n + 64,
                 storage="bf16")
    ora.prefill(0, k32.astype(np.float64), v32.astype(np.float64))
    la, na, ha, ua = _history(cfg_a, a)
    lb, nb, hb, ub = _history(cfg_b, b)
    assert (la, na) == (lb, nb) == (n, n - w.window - (n - w.window) % 64)
    worst_ora, worst_bb = 0.0, 0.0
    for u in range(len(ua)):
        ou = ora.unit(0, 0, u)
        for x, f in enumerate((ou.K, ou.V)):
            np.testing.assert_array_equal(ua[u][x]["basis"], ub[u][x]["basis"])
            np.testing.assert_array_equal(ua[u][x]["S"], ub[u][x]["S"])
            Ho = f.C[:na] @ f.B.T
            worst_ora = max(worst_ora, float(np.linalg.norm(ha[u][x] - Ho) / np.linalg.norm(Ho)))
            worst_bb = max(worst_bb, float(np.linalg.norm(ha[u][x] - hb[u][x]) / np.linalg.norm(hb[u][x])))
    q = q32(workloads.query(w, 0, 0))
    out_a = _decode(a, q, n - 1)
    err = rel_err_per_head(out_a, ora.decode_attn(0, q, n - 1))
    err_bb = rel_err_per_head(out_a, _decode(b, q, n - 1))
    a.destroy()
    b.destroy()
    print(f"prefill bf16 vs oracle: history {worst_ora:.2e}, outputs {err:.2e}; "
          f"vs block by block on the GPU: history {worst_bb:.2e}, outputs {err_bb:.2e}")
    assert worst_ora < 2e-3, worst_ora
    assert err < WALK_ENVELOPE[20][1], err


def test_prefill_state_errors():
    from rank_decode_attention_iskv_amd import binding
    w = small(1, kv_heads=2, q_heads=4, window=128)
    cfg, gpu = _cache(w, 1024, prefix=64)
    k, v = workloads.tokens(w, 0, 0, 512)
    kt, vt = _dev(k), _dev(v)
    with pytest.raises(binding.IskvError) as e:          # protected prefix not yet appended
        gpu.prefill(0, kt[:, :256], vt[:, :256])
    assert e.value.code == binding.ESTATE
    gpu.append(0, kt[:, :64], vt[:, :64])
    gpu.prefill(0, kt[:, 64:100], vt[:, 64:100])         # shorter than the window: all exact
    st = gpu.status(0)
    assert (st.length, st.compressed, st.folds) == (100, 0, 0)
    with pytest.raises(binding.IskvError) as e:          # ring not empty
        gpu.prefill(0, kt[:, 100:400], vt[:, 100:400])
    assert e.value.code == binding.ESTATE
    gpu.destroy()


def test_prefill_layers_matches_per_layer_prefill():
    """Three layers prefilled in one iskv_prefill_layers call (the M slots
    split three ways) against three single-layer calls: the same folds
    (bases, singular values bit-identical in fp32), the same history to fp32
    rounding of the deferred products."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = small(1, batch=2, kv_heads=2, q_heads=4, window=128, rank=16)
    n = 128 + 64 * 11 + 5
    storage = binding.F32
    cfg = binding.make_config(w.batch, 3, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, n + 64,
                              storage)
    a, b = binding.IskvCache(cfg), binding.IskvCache(cfg)
    ks, vs = [], []
    for layer in range(3):
        k, v = workloads.tokens(w, layer, 0, n)
        ks.append(_dev(k))
        vs.append(_dev(v))
    a.prefill_layers([0, 1, 2], ks, vs)
    for layer in range(3):
        b.prefill(layer, ks[layer], vs[layer])
    for layer in range(3):
        la, na, ua = binding.unpack_state(cfg, a.export_state(layer))
        lb, nb, ub = binding.unpack_state(cfg, b.export_state(layer))
        assert (la, na) == (lb, nb) == (n, 64 * 11)
        for xa, xb in zip(ua, ub):
            for fa, fb in zip(xa, xb):
                np.testing.assert_array_equal(fa["basis"], fb["basis"])
                np.testing.assert_array_equal(fa["S"], fb["S"])
                ha = fa["coef"][:na].astype(np.float64) @ fa["basis"].T
                hb = fb["coef"][:nb].astype(np.float64) @ fb["basis"].T
                assert np.linalg.norm(ha - hb) / np.linalg.norm(hb) < 1e-6
        assert a.status(layer).folds == 11
    a.destroy()
    b.destroy()
