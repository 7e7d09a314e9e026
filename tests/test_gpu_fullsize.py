"""Decode attention at the full workload sizes, GPU vs the float64 oracle.

The cache state is a random valid state of the workload's shapes (orthonormal
bases, coefficient rows, exact ring rows; bf16-grid values for bf16 storage),
imported into the library and installed in oracle units, so the full context
is checked without running the thousands of folds that would build it.  Every
query head of every sequence is compared (max relative 2-norm error 2e-3).

The launch configuration is the one bench.py times: the same library entry
point and split plan (single-round grids merge in the split kernel, larger
grids in the separate merge kernel; both occur below).
"""

import math

import numpy as np
import pytest

import workloads
from oracle import Unit
from tests.gpu_util import q32, rel_err_per_head

pytestmark = pytest.mark.gpu

ATOL_OUT = 2e-3


def _decode_vs_oracle(w, n_c, length, q_positions, rank_v=0):
    import torch
    from rank_decode_attention_iskv_amd import binding

    max_tokens = length + 64
    storage = binding.BF16 if w.storage == "bf16" else binding.F32
    cfg = binding.make_config(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              max_tokens, storage, rank_v=rank_v)
    gpu = binding.IskvCache(cfg)
    units = workloads.synthetic_state(w, length, n_c, max_tokens, rank_v=rank_v)
    gpu.import_state(0, binding.pack_state(cfg, length, n_c, units))
    st = gpu.status(0)
    assert (st.length, st.compressed) == (length, n_c)
    g = w.q_heads // w.kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    errs = []
    for step, q_pos in enumerate(q_positions):
        q = q32(workloads.query(w, 0, step))
        qt = torch.from_numpy(q.astype(np.float32)).cuda()
        out = torch.empty_like(qt)
        gpu.decode_attn(0, qt, q_pos, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = np.zeros_like(got)
        for ui, (xk, xv) in enumerate(units):
            b, h = divmod(ui, w.kv_heads)
            u = Unit(w.head_dim, w.rank, w.window, max_tokens, w.storage, r_v=rank_v or None)
            u.load_state(length, n_c, xk["ring"], xv["ring"], xk["basis"], xk["S"], xk["coef"],
                         xv["basis"], xv["S"], xv["coef"])
            ref[b, h * g:(h + 1) * g] = u.decode(q[b, h * g:(h + 1) * g], q_pos, scale)
        errs.append(rel_err_per_head(got, ref))
    gpu.destroy()
    return errs


def test_decode_full_size_gqa_layer_32k():
    """8 KV / 32 query heads, r = 32, window 256, bf16, 32K context (32512
    compressed + 277 exact tokens); the single-round grid merges in-kernel."""
    w = workloads.WORKLOADS[2]
    n_c = 32512
    errs = _decode_vs_oracle(w, n_c, n_c + w.window + 21, [n_c + w.window + 20, n_c + 400])
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs


def test_decode_full_size_batch16_16k_rank64():
    """Batch 16 x 16K, 8 KV / 32 query heads, r = 64, window 512, bf16; the
    multi-round grid uses the separate merge kernel."""
    w = workloads.WORKLOADS[3]
    n_c = 15872
    errs = _decode_vs_oracle(w, n_c, n_c + w.window + 45, [n_c + w.window + 44])
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs


@pytest.mark.parametrize("rank,n_extra", [(16, 0), (32, 63), (128, 1)])
def test_decode_window_bounds_and_ranks(rank, n_extra):
    """Exact region at its minimum (window) and maximum (window + 63) sizes,
    ranks 16 / 32 / 128, batch 4, on a 4K context."""
    w = workloads.with_(workloads.WORKLOADS[2], batch=4, rank=rank, window=128)
    n_c = 4096
    length = n_c + w.window + n_extra
    errs = _decode_vs_oracle(w, n_c, length, [length - 1, length + 150])
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs


@pytest.mark.parametrize("kv_heads,q_heads,batch", [(2, 12, 1), (1, 3, 1), (4, 12, 16), (8, 8, 1)])
def test_decode_many_splits_odd_group(kv_heads, q_heads, batch):
    """Groups of 6, 3 and 1 query heads.  Batch 1 merges in-kernel, over more
    than 128 split records per unit for the single KV head (past the records
    the merge keeps in registers); batch 16 (64 units) uses the merge kernel.
    r = 32, window 256, bf16, 16K context."""
    w = workloads.with_(workloads.WORKLOADS[2], batch=batch, kv_heads=kv_heads, q_heads=q_heads)
    n_c = 16384
    length = n_c + w.window + 7
    errs = _decode_vs_oracle(w, n_c, length, [length + 3])
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs


def test_decode_full_size_gqa_layer_32k_value_rank_64():
    """The 32K layer with a value rank twice the key rank (r_K = 32, r_V = 64),
    the configuration of bench.py --rank-v 64; single-round grid."""
    w = workloads.WORKLOADS[2]
    n_c = 32512
    errs = _decode_vs_oracle(w, n_c, n_c + w.window + 40, [n_c + w.window + 39, 77], rank_v=64)
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs


def test_decode_full_size_batch16_16k_rank32_value64():
    """Batch 16 x 16K, r_K = 32, r_V = 64, window 512: the multi-round grid
    with the separate merge kernel at the value rank."""
    w = workloads.with_(workloads.WORKLOADS[3], rank=32)
    n_c = 15872
    errs = _decode_vs_oracle(w, n_c, n_c + w.window + 3, [n_c + w.window + 2], rank_v=64)
    print(f"decode error on the same state: {max(errs):.2e}")
    assert max(errs) < ATOL_OUT, errs
