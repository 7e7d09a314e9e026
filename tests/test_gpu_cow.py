"""Copy-on-write maintenance (async_maintenance contexts) against the oracle.

Fold + sync run on a maintenance stream into the layer's second generation
while decode goes on over the current one; the switch happens at a decode
boundary once the maintenance has finished ["ASKV" design report, Design
requirements].  The oracle models this as a deferred fold: a ring with 64
rows of slack, the ready block folded when the GPU reports the switch (the
fold of a block commutes with appending later tokens; pinned on the CPU in
test_oracle_pins).  The maintenance stream is held back by a spin kernel
before some maintenances, so that decodes certainly run while one is in
flight.
"""

import numpy as np
import pytest

import workloads
from oracle import Oracle
from tests.gpu_util import q32, rel_err_per_head, small

pytestmark = pytest.mark.gpu


def _cache(w, layers, max_tokens, cow, rank_v=0, joint=False):
    from rank_decode_attention_iskv_amd import binding
    storage = binding.BF16 if w.storage == "bf16" else binding.F32
    cfg = binding.make_config(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim, w.rank,
                              w.window, max_tokens, storage, rank_v=rank_v,
                              async_maintenance=1 if cow else 0, joint_heads=int(joint))
    return cfg, binding.IskvCache(cfg)


def _step_tensors(w, layer, pos, step):
    import torch
    k, v = workloads.tokens(w, layer, pos, 1)
    q = q32(workloads.query(w, layer, step))
    return (k.astype(np.float32), v.astype(np.float32), q,
            torch.from_numpy(k.astype(np.float32)).cuda(),
            torch.from_numpy(v.astype(np.float32)).cuda(),
            torch.from_numpy(q.astype(np.float32)).cuda())


@pytest.mark.parametrize("rank,rank_v,joint", [(32, 0, False), (16, 32, False), (32, 64, True)])
def test_cow_decode_matches_deferred_oracle(rank, rank_v, joint):
    """fp32 storage, 2 sequences x 2 KV heads, 2 layers: every decode (fused
    append + attend) against the oracle folded exactly when the GPU switched
    (also with one basis per sequence over both heads)."""
    import torch
    w = small(1, batch=2, kv_heads=2, q_heads=8, window=128, rank=rank, shared_latent=joint)
    layers, tokens = 2, 128 + 64 * 7
    cfg, gpu = _cache(w, layers, tokens + 64, cow=True, rank_v=rank_v, joint=joint)
    ms = torch.cuda.Stream()
    gpu.set_maintenance_stream(ms)
    ora = Oracle(w.batch, layers, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window,
                 tokens + 64, storage=w.storage, rank_v=rank_v or None, slack=64,
                 joint_heads=joint)
    length = [0] * layers
    worst, in_flight_decodes, switches, held = 0.0, 0, 0, 0
    out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
    for step in range(tokens):
        for layer in range(layers):
            k, v, q, kt, vt, qt = _step_tensors(w, layer, length[layer], step)
            before = gpu.status(layer).compressed
            ready = gpu.append_decode(layer, kt, vt, qt, length[layer], out)
            st = gpu.status(layer)
            ora.append(layer, k.astype(np.float64), v.astype(np.float64))
            if st.compressed != before:
                assert st.compressed == before + 64
                ora.block_update(layer)
                ora.sync(layer)
                switches += 1
            got = out.cpu().numpy().astype(np.float64)
            ref = ora.decode_attn(layer, q, length[layer])
            worst = max(worst, rel_err_per_head(got, ref))
            in_flight_decodes += st.pending_sync
            length[layer] += 1
            if ready:
                if held % 2 == 0:
                    with torch.cuda.stream(ms):
                        torch.cuda._sleep(20_000_000)      # hold the maintenance back
                held += 1
                gpu.maintain(layer)
    gpu.join_maintenance()
    torch.cuda.synchronize()
    gpu.destroy()
    print(f"cow vs deferred oracle: worst {worst:.2e}, switches {switches}, "
          f"decodes during maintenance {in_flight_decodes}")
    assert worst < 1e-4, worst
    assert switches >= 2 * (tokens - 128 - 64) // 64 - 2
    assert in_flight_decodes >= 4


def _bf16_runs(layers=2, rounds=8):
    """The same stream through a copy-on-write context (switch forced right
    after each maintenance) and a plain one (block update + sync)."""
    import torch
    w = small(2, kv_heads=2, q_heads=8, window=128)
    max_tokens = 128 + 64 * (rounds + 2)
    runs = []
    for cow in (True, False):
        cfg, gpu = _cache(w, layers, max_tokens, cow)
        if cow:
            gpu.set_maintenance_stream(torch.cuda.Stream())
        outs, length = [], [0] * layers
        out = torch.empty(w.batch, w.q_heads, w.head_dim, device="cuda")
        for step in range(128 + 64 * rounds):
            for layer in range(layers):
                _, _, _, kt, vt, qt = _step_tensors(w, layer, length[layer], step)
                ready = gpu.append_decode(layer, kt, vt, qt, length[layer], out)
                outs.append(out.cpu().numpy().copy())
                length[layer] += 1
                if ready:
                    if cow:
                        gpu.maintain(layer)
                        assert gpu.switch(layer, wait=True)
                    else:
                        gpu.block_update(layer)
                        gpu.sync(layer)
        from rank_decode_attention_iskv_amd import binding
        states = [binding.unpack_state(cfg, gpu.export_state(l)) for l in range(layers)]
        assert gpu.status(0).folds == rounds
        gpu.destroy()
        runs.append((outs, states))
    return runs


def test_cow_forced_switch_is_bit_identical_to_in_place_bf16():
    """bf16: with the switch forced right after each maintenance, the
    copy-on-write path (fold and sync into the other generation) gives the
    same decode outputs and states, bit for bit, as the in-place path."""
    (oa, sa), (ob, sb) = _bf16_runs()
    for a, b in zip(oa, ob):
        np.testing.assert_array_equal(a, b)
    for (la, na, ua), (lb, nb, ub) in zip(sa, sb):
        assert (la, na) == (lb, nb)
        for xa, xb in zip(ua, ub):
            for fa, fb in zip(xa, xb):
                np.testing.assert_array_equal(fa["basis"], fb["basis"])
                np.testing.assert_array_equal(fa["S"], fb["S"])
                np.testing.assert_array_equal(fa["coef"], fb["coef"])


def test_cow_state_machine():
    """Verbs that do not belong to the mode are refused; maintain needs a
    ready block and no maintenance in flight; a full ring waits for the switch."""
    import torch
    from rank_decode_attention_iskv_amd import binding
    w = small(1, kv_heads=2, q_heads=4, window=128)
    cfg, gpu = _cache(w, 1, 512, cow=True)
    plain_cfg, plain = _cache(w, 1, 512, cow=False)
    with pytest.raises(binding.IskvError) as e:
        plain.maintain(0)
    assert e.value.code == binding.ESTATE
    plain.destroy()
    k, v = workloads.tokens(w, 0, 0, 256)
    kt, vt = torch.from_numpy(k.astype(np.float32)).cuda(), torch.from_numpy(v.astype(np.float32)).cuda()
    with pytest.raises(binding.IskvError) as e:
        gpu.maintain(0)                                  # nothing ready
    assert e.value.code == binding.ESTATE
    assert gpu.append(0, kt[:, :192], vt[:, :192])       # window + 64 rows: ready
    for verb in (gpu.block_update, gpu.sync, gpu.discard_sync):
        with pytest.raises(binding.IskvError) as e:
            verb(0)
        assert e.value.code == binding.ESTATE
    gpu.maintain(0)
    with pytest.raises(binding.IskvError) as e:
        gpu.maintain(0)                                  # one in flight
    assert e.value.code == binding.ESTATE
    st = gpu.status(0)
    assert (st.compressed, st.pending_sync, st.blocks_ready) in ((0, 1, 0), (64, 0, 0))
    # 64 more rows fit in the slack; the next would overflow and waits for the switch
    gpu.append(0, kt[:, 192:256], vt[:, 192:256])
    assert gpu.append(0, kt[:, :1], vt[:, :1]) in (False, True)
    st = gpu.status(0)
    assert (st.length, st.compressed, st.pending_sync) == (257, 64, 0)
    gpu.destroy()
