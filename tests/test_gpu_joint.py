"""Joint-head basis on the GPU against the oracle's JointUnit.

One basis per (sequence, layer) and factor over all KV heads (rows of
kv_heads * 128), one coefficient row per token for all heads [iS-KV
explainer, the worked example and Table 1: ranks 64-128 compress 128-dim
heads 4-7x, which needs a basis over several heads].  The inputs come from
workloads with shared_latent=True: the heads of a (sequence, layer) mix the
same latent factors, so their stacked rows are low-rank.
"""

from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.gpu_util import Pair, exact_attention, q32, rel_err_per_head, small, subspace_dist

pytestmark = pytest.mark.gpu

ATOL_OUT = 2e-3


def _joint(wid, **kw):
    return small(wid, shared_latent=True, **kw)


def _oracle_joint(w, L, fold_last=True, rank_v=None):
    """Joint oracle state after L tokens (fold + sync each time the ring
    fills); fold_last=False leaves a full ring at the end unfolded."""
    from oracle import Oracle
    o = Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, L + 128,
               storage=w.storage, rank_v=rank_v, joint_heads=True)
    pos = 0
    u0 = o.unit(0, 0, 0)
    while pos < L:
        n = min(64, L - pos, w.window + 64 - (u0.length - u0.n_c))
        k, v = workloads.tokens(w, 0, pos, n)
        ready = o.append(0, k.astype(np.float32).astype(np.float64),
                         v.astype(np.float32).astype(np.float64))
        pos += n
        if ready and (fold_last or pos < L):
            o.block_update(0)
            o.sync(0)
    return o


def _joint_basis(units, b, H, x):
    """A sequence's joint basis (H*d x r) from the per-head slices of a state."""
    return np.concatenate([units[b * H + h][x]["basis"].astype(np.float64) for h in range(H)])


def _leading(s):
    """Gapped leading count: largest k with s_k / s_(k+1) >= 10, else the
    directions above 1e-3 s_1."""
    r = len(s)
    gaps = [k for k in range(1, r) if s[k] > 0 and s[k - 1] / s[k] >= 10]
    return gaps[-1] if gaps else int(np.sum(s > 1e-3 * s[0]))


@pytest.mark.parametrize("kw,folds,rank_v", [
    (dict(storage="f32", rank=32, signal_rank=24, window=128), 4, 0),
    (dict(storage="f32", rank=64, signal_rank=48, window=64, batch=2), 3, 0),
    (dict(storage="f32", rank=16, signal_rank=12, kv_heads=4, q_heads=16, window=64), 5, 32),
    (dict(storage="bf16", rank=64, signal_rank=48, window=128), 6, 0),
    (dict(storage="bf16", rank=32, signal_rank=32, window=64, batch=2), 3, 64),
])
def test_joint_fold_and_sync_on_imported_oracle_state(kw, folds, rank_v):
    """One block update + sync of every (sequence, K|V) on an identical
    joint state: basis orthonormal, leading subspace (f32) and S, the rebuilt
    history of all heads, and decode of every query head."""
    w = _joint(2, **kw)
    H = w.kv_heads
    L = w.window + 64 * (folds + 1)
    o = _oracle_joint(w, L, fold_last=False, rank_v=rank_v or None)
    p = Pair(w, max_tokens=L + 128, oracle=False, rank_v=rank_v, joint=True)
    p.ora = o
    p.gpu.import_state(0, p.oracle_blob(0))
    assert p.gpu.status(0).blocks_ready == 1
    p.gpu.block_update(0)
    p.gpu.sync(0)
    o.block_update(0)
    o.sync(0)
    length, n_c, units = p.state(0)
    assert (length, n_c) == (o.unit(0, 0, 0).length, o.unit(0, 0, 0).n_c)
    for b in range(w.batch):
        ou = o.unit(b, 0, 0)
        for x, f in enumerate((ou.K, ou.V)):
            B = _joint_basis(units, b, H, x)
            r = B.shape[1]
            assert B.shape == (H * w.head_dim, r)
            assert np.linalg.norm(B.T @ B - np.eye(r), 2) < 1e-5
            k = _leading(f.S)
            if w.storage == "f32":
                assert subspace_dist(B[:, :k], f.B[:, :k]) < 1e-4
            Sg = units[b * H][x]["S"]
            np.testing.assert_allclose(Sg[:k], f.S[:k], rtol=1e-4, atol=1e-5 * f.S[0])
            # every head lists the same S and coefficient rows
            for h in range(1, H):
                np.testing.assert_array_equal(units[b * H + h][x]["S"], Sg)
                np.testing.assert_array_equal(units[b * H + h][x]["coef"][:n_c],
                                              units[b * H][x]["coef"][:n_c])
            H_gpu = units[b * H][x]["coef"][:n_c].astype(np.float64) @ B.T
            H_ora = f.C[:n_c] @ f.B.T
            err = np.linalg.norm(H_gpu - H_ora) / np.linalg.norm(H_ora)
            print(f"joint {w.storage} r={r} history error {err:.2e}")
            assert err < (1e-4 if w.storage == "f32" else 1e-3)
    for step, q_pos in enumerate([L - 1, L + 3]):
        q = q32(workloads.query(w, 0, step))
        got = p.decode(0, q, q_pos)
        ref = o.decode_attn(0, q, q_pos)
        err = rel_err_per_head(got, ref)
        print(f"joint {w.storage} decode error {err:.2e}")
        assert err < ATOL_OUT


@pytest.mark.parametrize("kw,L,rank_v", [
    (dict(storage="f32", rank=32, signal_rank=24, noise_std=0.01, window=128), 64 * 12 + 128 + 21, 0),
    (dict(storage="f32", rank=64, signal_rank=64, spectrum="power", noise_std=0.0, window=64,
          batch=2), 64 * 8 + 64 + 40, 0),
    (dict(storage="f32", rank=32, signal_rank=32, window=64, kv_heads=4, q_heads=8), 64 * 9 + 64 + 3, 64),
])
def test_joint_end_to_end_fp32(kw, L, rank_v):
    """Appends, folds and syncs through the library against the joint oracle
    fed the same stream: states and decode at several points."""
    w = _joint(2, **kw)
    H = w.kv_heads
    p = Pair(w, max_tokens=L + 128, rank_v=rank_v, joint=True)
    checks = []

    def on_fold(pp):
        st = pp.gpu.status(0)
        if st.compressed // 64 in (1, 3):
            q = q32(workloads.query(w, 0, 100 + st.compressed))
            checks.append(rel_err_per_head(pp.decode(0, q, st.length - 1),
                                           pp.ora.decode_attn(0, q, st.length - 1)))
    p.feed(0, L, on_fold=on_fold)
    length, n_c, units = p.state(0)
    for b in range(w.batch):
        ou = p.ora.unit(b, 0, 0)
        assert (length, n_c) == (ou.length, ou.n_c)
        for x, f in enumerate((ou.K, ou.V)):
            B = _joint_basis(units, b, H, x)
            assert np.linalg.norm(B.T @ B - np.eye(B.shape[1]), 2) < 1e-5
            H_gpu = units[b * H][x]["coef"][:n_c].astype(np.float64) @ B.T
            H_ora = f.C[:n_c] @ f.B.T
            assert np.linalg.norm(H_gpu - H_ora) / np.linalg.norm(H_ora) < 1e-3
    for step, q_pos in enumerate([L - 1, L]):
        q = q32(workloads.query(w, 0, step))
        checks.append(rel_err_per_head(p.decode(0, q, q_pos), p.ora.decode_attn(0, q, q_pos)))
    print("joint f32 end-to-end decode errors", ["%.2e" % e for e in checks])
    assert len(checks) >= 3 and max(checks) < ATOL_OUT


def test_joint_lossless_is_exact_attention_fp32():
    """Noise-free shared-latent data of rank 24 over 8 heads, joint r = 32:
    every fold keeps the heads' rows, so decode is exact attention per head,
    while each head alone would need rank 24 of its own."""
    w = _joint(2, storage="f32", rank=32, signal_rank=24, noise_std=0.0, window=64)
    L = 64 * 10 + 64 + 11
    p = Pair(w, max_tokens=L + 64, oracle=False, joint=True)
    p.feed(0, L)
    assert p.gpu.status(0).compressed == 640
    for step, q_pos in enumerate([L - 1, L + 5]):
        q = q32(workloads.query(w, 0, step))
        err = rel_err_per_head(p.decode(0, q, q_pos), exact_attention(w, L, q, q_pos))
        print(f"joint lossless: error vs exact attention {err:.2e}")
        assert err < 1e-4


def test_joint_bf16_quality_against_exact_attention():
    """bf16 storage, 16 joint folds through the GPU: the error against
    uncompressed attention is no worse than the oracle's (bf16 mirror)."""
    w = _joint(2, storage="bf16", rank=64, signal_rank=48, window=128)
    L = 64 * 16 + 128 + 30
    p = Pair(w, max_tokens=L + 64, joint=True)
    p.feed(0, L)
    for step in range(2):
        q = q32(workloads.query(w, 0, step))
        got = p.decode(0, q, L - 1)
        ora = p.ora.decode_attn(0, q, L - 1)
        exact = exact_attention(w, L, q, L - 1)
        e_gpu, e_ora = rel_err_per_head(got, exact), rel_err_per_head(ora, exact)
        print(f"joint bf16: vs exact gpu {e_gpu:.2e} oracle {e_ora:.2e}; gpu vs oracle "
              f"{rel_err_per_head(got, ora):.2e}")
        assert e_gpu < 1.5 * e_ora + 2e-3, (e_gpu, e_ora)


def test_joint_protected_prefix_fp32():
    """A protected prefix of 128 exact positions with a joint basis after it."""
    w = _joint(2, storage="f32", rank=32, signal_rank=24, window=64, kv_heads=4, q_heads=8)
    L = 128 + 64 * 6 + 64 + 9
    p = Pair(w, max_tokens=L + 64, prefix=128, joint=True)
    p.feed(0, L)
    st = p.gpu.status(0)
    assert st.compressed == p.ora.unit(0, 0, 0).compressed > 0
    for step, q_pos in enumerate([L - 1, L + 2]):
        q = q32(workloads.query(w, 0, step))
        assert rel_err_per_head(p.decode(0, q, q_pos), p.ora.decode_attn(0, q, q_pos)) < ATOL_OUT


def test_joint_ragged_fp32():
    """Ragged batch of two sequences with a joint basis: per-sequence
    lengths and folds against the oracle's joint unit of each sequence."""
    import torch
    from oracle import JointUnit
    w = _joint(2, storage="f32", rank=32, signal_rank=24, window=64, kv_heads=4, q_heads=8, batch=2)
    H, d = w.kv_heads, w.head_dim
    lens = [64 * 7 + 64 + 5, 64 * 3 + 64 + 40]
    p = Pair(w, max_tokens=max(lens) + 128, oracle=False, joint=True)
    ora = [JointUnit(H, d, w.rank, w.window, max(lens) + 128, "f32") for _ in range(2)]
    k_all, v_all = workloads.tokens(w, 0, 0, max(lens))
    k_all, v_all = k_all.astype(np.float32), v_all.astype(np.float32)
    pos = [0, 0]
    while pos != lens:
        n = [min(48, lens[b] - pos[b], w.window + 64 - (ora[b].length - ora[b].n_c)) for b in range(2)]
        kb = np.zeros((2, max(max(n), 1), H, d), np.float32)
        vb = np.zeros_like(kb)
        for b in range(2):
            kb[b, :n[b]] = k_all[b, pos[b]:pos[b] + n[b]]
            vb[b, :n[b]] = v_all[b, pos[b]:pos[b] + n[b]]
            for t in range(n[b]):
                ora[b].append(kb[b, t].astype(np.float64), vb[b, t].astype(np.float64))
            pos[b] += n[b]
        p.gpu.append_ragged(0, torch.from_numpy(kb).cuda(), torch.from_numpy(vb).cuda(), n)
        if any(u.ready for u in ora):
            p.gpu.block_update(0)
            p.gpu.sync(0)
            for u in ora:
                if u.ready:
                    u.fold()
                    u.sync()
    for b in range(2):
        st = p.gpu.seq_status(0, b)
        assert (st.length, st.compressed) == (ora[b].length, ora[b].n_c)
    q = q32(workloads.query(w, 0, 0))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out = torch.empty_like(qt)
    p.gpu.decode_attn_ragged(0, qt, [lens[0] - 1, lens[1] + 2], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = np.stack([ora[0].decode(q[0], lens[0] - 1, 1 / np.sqrt(d)),
                    ora[1].decode(q[1], lens[1] + 2, 1 / np.sqrt(d))])
    assert rel_err_per_head(got, ref) < ATOL_OUT


def test_joint_config_and_state_errors():
    """Joint contexts refuse bulk prefill; their byte count keeps one
    coefficient row per token for all heads."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = _joint(2, storage="bf16", rank=64, signal_rank=48, window=64)
    p = Pair(w, max_tokens=1024, oracle=False, joint=True)
    k, v = workloads.tokens(w, 0, 0, 256)
    with pytest.raises(binding.IskvError) as e:
        p.gpu.prefill(0, torch.from_numpy(k.astype(np.float32)).cuda(),
                      torch.from_numpy(v.astype(np.float32)).cuda())
    assert e.value.code == binding.ESTATE
    p.feed(0, 64 * 4 + 64 + 10)
    st = p.gpu.status(0)
    from oracle import persistent_kv_bytes
    n_e = st.length - st.compressed
    assert st.persistent_bytes == persistent_kv_bytes(st.compressed, n_e, 1, w.kv_heads, w.head_dim,
                                                      w.rank, 2, joint_heads=True)


def _joint_full_size(w, n_c, length, q_positions, sample, fold=False):
    """A random joint state of the workload's full shapes imported into the
    library; decode (and, with fold=True, one block update + sync first) of
    every sequence, compared with the joint oracle on the sampled sequences."""
    import math

    import torch
    from oracle import JointUnit
    from rank_decode_attention_iskv_amd import binding

    H, d = w.kv_heads, w.head_dim
    max_tokens = length + 64
    cfg = binding.make_config(w.batch, 1, H, w.q_heads, d, w.rank, w.window, max_tokens,
                              binding.BF16 if w.storage == "bf16" else binding.F32, joint_heads=1)
    gpu = binding.IskvCache(cfg)
    states = {}

    def units():
        for b in range(w.batch):
            xs = workloads.synthetic_joint(w, b, length, n_c, max_tokens, ring_in_span=fold)
            if b in sample:
                states[b] = xs
            for h in range(H):
                cols = slice(h * d, (h + 1) * d)
                yield [dict(basis=x["basis"][cols], S=x["S"], coef=x["coef"], ring=x["ring"][:, cols])
                       for x in xs]
    gpu.import_state(0, binding.pack_state(cfg, length, n_c, units()))
    oras = {}
    for b in sample:
        xk, xv = states[b]
        u = JointUnit(H, d, w.rank, w.window, max_tokens, w.storage)
        u.load_state(length, n_c, xk["ring"], xv["ring"], xk["basis"], xk["S"], xk["coef"],
                     xv["basis"], xv["S"], xv["coef"])
        oras[b] = u
    if fold:
        assert gpu.status(0).blocks_ready == 1
        gpu.block_update(0)
        gpu.sync(0)
        for u in oras.values():
            u.fold()
            u.sync()
        length2, n_c2, st = binding.unpack_state(cfg, gpu.export_state(0))
        for b, u in oras.items():
            for x, f in enumerate((u.K, u.V)):
                B = np.concatenate([st[b * H + h][x]["basis"].astype(np.float64) for h in range(H)])
                assert np.linalg.norm(B.T @ B - np.eye(B.shape[1]), 2) < 1e-5
                k = _leading(f.S)
                np.testing.assert_allclose(st[b * H][x]["S"][:k], f.S[:k], rtol=1e-4, atol=1e-5 * f.S[0])
                H_gpu = st[b * H][x]["coef"][:n_c2].astype(np.float64) @ B.T
                H_ora = f.C[:n_c2] @ f.B.T
                err = np.linalg.norm(H_gpu - H_ora) / np.linalg.norm(H_ora)
                print(f"joint full-size fold: sequence {b} history error {err:.2e}")
                assert err < 1e-3
    g = w.q_heads // H
    errs = []
    for step, q_pos in enumerate(q_positions):
        q = q32(workloads.query(w, 0, step))
        qt = torch.from_numpy(q.astype(np.float32)).cuda()
        out = torch.empty_like(qt)
        gpu.decode_attn(0, qt, q_pos, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        for b, u in oras.items():
            ref = u.decode(q[b], q_pos, 1.0 / math.sqrt(d))
            errs.append(rel_err_per_head(got[b:b + 1], ref[None]))
    gpu.destroy()
    print("joint full-size decode errors", ["%.2e" % e for e in errs])
    return errs


def test_joint_full_size_batch16_16k_rank64():
    """Batch 16 x 16K, 8 KV / 32 query heads, one basis per sequence over the
    8 heads at r = 64, window 512, bf16 (the joint bench preset's shapes):
    decode of all sequences, sequences 0, 7 and 15 against the oracle."""
    w = workloads.with_(workloads.WORKLOADS[3], shared_latent=True)
    n_c = 15872
    errs = _joint_full_size(w, n_c, n_c + w.window + 45, [n_c + w.window + 44], sample=(0, 7, 15))
    assert max(errs) < ATOL_OUT, errs


def test_joint_full_size_gqa_layer_32k_fold_and_sync():
    """The 32K GQA layer with a joint basis at r = 64 (bf16): one block
    update + sync at full length, then decode, against the oracle."""
    w = workloads.with_(workloads.WORKLOADS[2], rank=64, shared_latent=True)
    n_c = 32448
    length = n_c + w.window + 64              # ring full: the next fold is ready
    errs = _joint_full_size(w, n_c, length, [length - 1, length + 5], sample=(0,), fold=True)
    assert max(errs) < ATOL_OUT, errs
