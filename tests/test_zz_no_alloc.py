"""The allocation-free decode entry point (iskv_decode_attn_noalloc) against
iskv_decode_attn: same kernels and plan, split records in the library's static
device array instead of the workspace, so the outputs must be bit-identical.
Two calls in a row, the second on a smaller input (a shorter layer of a
second context), plus the size limit."""

import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_util import q32

pytestmark = pytest.mark.gpu


def _cache(w, length, n_c, layers=1):
    from rank_decode_attention_iskv_amd import binding
    max_tokens = length + 64
    cfg = binding.make_config(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                              max_tokens, binding.BF16)
    gpu = binding.IskvCache(cfg)
    gen = (workloads.synthetic_unit(w, b, h, length, n_c, max_tokens)
           for b in range(w.batch) for h in range(w.kv_heads))
    gpu.import_state(0, binding.pack_state(cfg, length, n_c, gen))
    return cfg, gpu


def _both(gpu, q, q_pos):
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).cuda()
    a, b = torch.empty_like(qt), torch.full_like(qt, float("nan"))
    gpu.decode_attn(0, qt, q_pos, a)
    gpu.decode_attn_noalloc(0, qt, q_pos, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_decode_matches_workspace_decode_twice():
    # first call: the 32K GQA layer (8 KV / 32 query heads, r = 32, bf16)
    w = workloads.WORKLOADS[2]
    n_c = 32512
    cfg, gpu = _cache(w, n_c + w.window + 21, n_c)
    q = q32(workloads.query(w, 0, 0))
    ref, got = _both(gpu, q, n_c + w.window + 20)
    assert np.all(np.isfinite(got))
    np.testing.assert_array_equal(got, ref)
    # second call, smaller input: batch 2 x 2 KV heads at 4K (a merge over
    # fewer records, leaving the first call's records behind in the array)
    w2 = workloads.with_(w, batch=2, kv_heads=2, q_heads=8, window=128)
    cfg2, gpu2 = _cache(w2, 4096 + 128 + 5, 4096)
    q2 = q32(workloads.query(w2, 0, 1))
    ref2, got2 = _both(gpu2, q2, 4096 + 128 + 4)
    assert np.all(np.isfinite(got2))
    np.testing.assert_array_equal(got2, ref2)
    # and the first context again, after the smaller one
    ref3, got3 = _both(gpu, q, n_c + 300)
    np.testing.assert_array_equal(got3, ref3)
    gpu.destroy()
    gpu2.destroy()


def test_noalloc_rejects_configurations_beyond_its_array():
    """A configuration whose split records exceed the static array: the call
    fails on the host with ISKV_ESCRATCH, before any launch."""
    from rank_decode_attention_iskv_amd import binding
    cfg = binding.make_config(300, 1, 8, 128, 128, 32, 64, 256, binding.BF16)
    assert binding.noalloc_scratch_bytes(cfg) > (32 << 20)
    gpu = binding.IskvCache(cfg)
    import torch
    k = torch.randn(300, 64, 8, 128, device="cuda")
    gpu.append(0, k, k)
    q = torch.randn(300, 128, 128, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(binding.IskvError) as e:
        gpu.decode_attn_noalloc(0, q, 63, out)
    assert e.value.code == binding.ESCRATCH
    gpu.destroy()
