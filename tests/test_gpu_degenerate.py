"""Degenerate blocks through the GPU fold, against the float64 oracle and
against closed forms that do not depend on it.

  * all-zero keys: every folded key block is zero, so the key core has no
    non-zero singular value, the residual pivots all fall under the guard and
    the key basis is made of completed null directions (iS-KV explainer,
    Block-incremental SVD: the fold of a block into the basis).  Every score
    is then 0 and attention is the plain mean of the values; with noise-free
    values of rank 12 < r in fp32 the compressed values are exact, so the
    output is the mean of the raw value rows.
  * repeated tokens: each 64-token block repeats one key row, so each block
    has rank 1 and the residual Gram has a single non-zero pivot.  Seven
    distinct keys fit in r = 32: the key history comes back exactly.
  * the shortest caches (1, 2, 15, 16, 17 and 33 tokens, all in the exact
    window, one partly filled 16-token tile): against the oracle, and at one
    token against softmax over a single key, which returns that token's value.
"""

import numpy as np
import pytest

import workloads
from oracle import Oracle
from tests.gpu_util import Pair, q32, rel_err_per_head, small

pytestmark = pytest.mark.gpu

ATOL_OUT = 2e-3


def _run(w, k, v, max_tokens):
    """Feed k, v ([batch, L, kv_heads, d]) to a GPU cache and the oracle in
    64-token chunks, folding and syncing whenever the ring fills."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    storage = binding.BF16 if w.storage == "bf16" else binding.F32
    cfg = binding.make_config(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              max_tokens, storage)
    gpu = binding.IskvCache(cfg)
    ora = Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, max_tokens,
                 storage=w.storage)
    L = k.shape[1]
    done = folds = 0
    slots = w.window + 64
    while done < L:
        st = gpu.status(0)
        free = slots - (st.length - st.compressed)
        n = min(64, free, L - done)
        k32 = np.ascontiguousarray(k[:, done:done + n], dtype=np.float32)
        v32 = np.ascontiguousarray(v[:, done:done + n], dtype=np.float32)
        ready = gpu.append(0, torch.from_numpy(k32).cuda(), torch.from_numpy(v32).cuda())
        ora.append(0, k32.astype(np.float64), v32.astype(np.float64))
        done += n
        if ready:
            gpu.block_update(0)
            gpu.sync(0)
            ora.block_update(0)
            ora.sync(0)
            folds += 1
    return cfg, gpu, ora, folds


def _decode(gpu, q, q_pos):
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    out = torch.empty_like(qt)
    gpu.decode_attn(0, qt, q_pos, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_zero_keys_give_the_mean_of_the_values(storage):
    w = small(1, window=64, signal_rank=12, noise_std=0.0, storage=storage)
    L = 64 * 6 + 64 + 5
    _, v = workloads.tokens(w, 0, 0, L)
    v = v.astype(np.float32).astype(np.float64)
    k = np.zeros_like(v)
    cfg, gpu, ora, folds = _run(w, k, v, L + 64)
    assert folds == 6
    from rank_decode_attention_iskv_amd import binding
    _, n_c, units = binding.unpack_state(cfg, gpu.export_state(0))
    assert gpu.status(0).numeric_flags == 0
    Bk, Ck = units[0][0]["basis"].astype(np.float64), units[0][0]["coef"][:n_c]
    assert np.all(np.isfinite(Bk)) and np.all(Ck == 0.0)
    assert np.linalg.norm(Bk.T @ Bk - np.eye(w.rank), 2) < 1e-5
    q = q32(workloads.query(w, 0, 0))
    got = _decode(gpu, q, L - 1)
    gpu.destroy()
    ref = ora.decode_attn(0, q, L - 1)
    err_ora = rel_err_per_head(got, ref)
    if storage == "f32":
        mean = v[:, :, 0].mean(axis=1)                     # [batch, d]
        err_mean = rel_err_per_head(got, np.broadcast_to(mean[:, None, :], got.shape))
    else:
        err_mean = float("nan")
    print(f"zero keys {storage}: vs oracle {err_ora:.2e}, vs mean of the values {err_mean:.2e}")
    assert err_ora < ATOL_OUT, err_ora
    if storage == "f32":
        assert err_mean < 1e-4, err_mean


def test_repeated_token_blocks_keep_the_key_history():
    w = small(1, window=64, signal_rank=12, noise_std=0.0)
    assert w.storage == "f32"
    L = 64 * 6 + 64 + 5
    k, v = workloads.tokens(w, 0, 0, L)
    k = k.astype(np.float32).astype(np.float64)
    v = v.astype(np.float32).astype(np.float64)
    for s in range(0, L, 64):
        k[:, s:s + 64] = k[:, s:s + 1]                     # one key row per 64-token block
    cfg, gpu, ora, folds = _run(w, k, v, L + 64)
    assert folds == 6
    from rank_decode_attention_iskv_amd import binding
    _, n_c, units = binding.unpack_state(cfg, gpu.export_state(0))
    assert gpu.status(0).numeric_flags == 0
    Bk = units[0][0]["basis"].astype(np.float64)
    Hk = units[0][0]["coef"][:n_c].astype(np.float64) @ Bk.T
    X = k[0, :n_c, 0]
    hist = float(np.linalg.norm(Hk - X) / np.linalg.norm(X))
    assert np.linalg.norm(Bk.T @ Bk - np.eye(w.rank), 2) < 1e-5
    errs = []
    for step, q_pos in enumerate([L - 1, L + 40]):
        q = q32(workloads.query(w, 0, step))
        errs.append(rel_err_per_head(_decode(gpu, q, q_pos), ora.decode_attn(0, q, q_pos)))
    gpu.destroy()
    print(f"repeated-token blocks: key history {hist:.2e}, decode vs oracle {max(errs):.2e}")
    assert hist < 1e-4, hist
    assert max(errs) < ATOL_OUT, errs


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_decode_on_the_shortest_caches(storage):
    w = small(2, kv_heads=2, q_heads=8, window=128, storage=storage)
    p = Pair(w, max_tokens=512)
    errs = {}
    for L in (1, 2, 15, 16, 17, 33):
        p.feed(0, L - p.length[0])
        q = q32(workloads.query(w, 0, L))
        got = p.decode(0, q, L - 1)
        errs[L] = rel_err_per_head(got, p.ora.decode_attn(0, q, L - 1))
        if L == 1 and storage == "f32":
            _, v0 = workloads.tokens(w, 0, 0, 1)
            g = w.q_heads // w.kv_heads
            v0 = v0[:, 0].astype(np.float32).astype(np.float64)       # [batch, kv_heads, d]
            one = np.repeat(v0, g, axis=1)                           # query head -> its KV head
            assert rel_err_per_head(got, one) < 1e-6
    print(f"shortest caches {storage}: " + ", ".join(f"L={L} {e:.1e}" for L, e in errs.items()))
    assert max(errs.values()) < ATOL_OUT, errs
