"""Host-only checks of the C-ABI library: it loads, exports every symbol the
header declares, and validates configurations without touching a GPU."""

import ctypes
import os
import re

import pytest

from rank_decode_attention_iskv_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "iskv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(iskv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = binding.load_library()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTED)


def base_cfg(**kw):
    d = dict(batch=2, num_layers=3, num_kv_heads=8, num_q_heads=32, head_dim=128, rank=32,
             window=256, max_tokens=4096, storage=binding.BF16)
    d.update(kw)
    return binding.make_config(**d)


def test_workspace_bytes_valid_and_monotone():
    small = binding.workspace_bytes(base_cfg())
    big = binding.workspace_bytes(base_cfg(max_tokens=8192))
    assert small > 0 and big > small
    # coefficients dominate: two factors x units x tokens x rank x 2 bytes per layer
    assert big - small >= 3 * 2 * 16 * 4096 * 32 * 2
    assert binding.workspace_bytes(base_cfg(storage=binding.F32)) > small


@pytest.mark.parametrize("kw", [
    dict(head_dim=64), dict(rank=48), dict(rank=256), dict(window=100), dict(window=0),
    dict(block=32), dict(num_q_heads=12), dict(num_q_heads=136), dict(storage=7),
    dict(batch=0), dict(max_tokens=0), dict(rope_base=0.5),
    dict(protected_prefix=100), dict(protected_prefix=-64), dict(protected_prefix=4160),
    dict(rank_v=48), dict(rank_v=16), dict(rank_v=-32), dict(rank=128, rank_v=256),
    dict(joint_heads=2), dict(joint_heads=1, rank=128), dict(joint_heads=1, rank=64, rank_v=128),
    dict(joint_heads=1, num_kv_heads=64, num_q_heads=64),
])
def test_invalid_configs_rejected(kw):
    assert binding.workspace_bytes(base_cfg(**kw)) == 0
    assert binding.state_bytes(base_cfg(**kw)) == 0


def test_state_bytes_layout():
    cfg = base_cfg(batch=1, num_kv_heads=2, num_q_heads=2, max_tokens=1000)
    d, r, T, S = 128, 32, 1000, 256 + 64
    assert binding.state_bytes(cfg) == 16 + 2 * 2 * (d * r + r + T * r + S * d) * 4
    # the protected prefix adds its exact rows per (unit, K|V)
    cfg = base_cfg(batch=1, num_kv_heads=2, num_q_heads=2, max_tokens=1000, protected_prefix=192)
    assert binding.state_bytes(cfg) == 16 + 2 * 2 * (d * r + r + T * r + S * d + 192 * d) * 4


def test_state_bytes_separate_v_rank():
    """With rank_v the V factor's basis, singular values and coefficients take
    r_V columns; rank_v equal to rank is the same as rank_v = 0."""
    d, T, S = 128, 1000, 256 + 64
    cfg = base_cfg(batch=1, num_kv_heads=2, num_q_heads=2, max_tokens=1000, rank_v=64)
    per_k = d * 32 + 32 + T * 32 + S * d
    per_v = d * 64 + 64 + T * 64 + S * d
    assert binding.state_bytes(cfg) == 16 + 2 * (per_k + per_v) * 4
    same = base_cfg(batch=1, num_kv_heads=2, num_q_heads=2, max_tokens=1000, rank_v=32)
    assert binding.state_bytes(same) == binding.state_bytes(
        base_cfg(batch=1, num_kv_heads=2, num_q_heads=2, max_tokens=1000))
    # workspace grows by at least the extra V coefficients (storage dtype)
    a = binding.workspace_bytes(base_cfg())
    b = binding.workspace_bytes(base_cfg(rank_v=64))
    assert b - a >= 3 * 16 * 4096 * 32 * 2


def test_protected_prefix_workspace():
    """The prefix rows (K and V, storage dtype) add at least 2 x units x P x d
    elements per layer to the workspace."""
    a = binding.workspace_bytes(base_cfg())
    b = binding.workspace_bytes(base_cfg(protected_prefix=512))
    assert b - a >= 3 * 2 * 16 * 512 * 128 * 2


def test_init_rejects_bad_arguments_without_device_work():
    lib = binding.load_library()
    ctx = ctypes.c_void_p()
    bad = base_cfg(rank=48)
    assert lib.iskv_init(ctypes.byref(bad), ctypes.c_void_p(256), 1 << 30, None,
                         ctypes.byref(ctx)) == binding.EINVAL
    good = base_cfg()
    # misaligned workspace pointer
    assert lib.iskv_init(ctypes.byref(good), ctypes.c_void_p(8), 1 << 40, None,
                         ctypes.byref(ctx)) == binding.EINVAL
    # null context for every verb
    assert lib.iskv_block_update(None, 0) == binding.EINVAL
    assert lib.iskv_sync(None, 0) == binding.EINVAL
    assert lib.iskv_destroy(None) == binding.EINVAL


def test_strerror_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert binding.strerror(code)
    assert binding.strerror(99) == "unknown error"


def test_joint_heads_workspace():
    """A joint basis keeps one coefficient row per token for all heads: the
    coefficient arrays shrink by the head count (the fold adds its scratch of
    64 + r rows of heads x d floats per sequence and factor)."""
    per_head = binding.workspace_bytes(base_cfg(rank=64))
    joint = binding.workspace_bytes(base_cfg(rank=64, joint_heads=1))
    assert joint > 0
    coef_per_head = 3 * 2 * 16 * 4096 * 64 * 2       # layers x factors x units x tokens x r x bf16
    scratch = 3 * 2 * 2 * (64 + 64) * 8 * 128 * 4    # layers x factors x sequences x rows x H*d x f32
    assert per_head - joint >= coef_per_head * 7 // 8 - scratch - (1 << 16)
    # the state blob keeps its per-head layout
    assert binding.state_bytes(base_cfg(rank=64, joint_heads=1)) == binding.state_bytes(base_cfg(rank=64))
