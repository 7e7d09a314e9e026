"""Pins of the float64 oracle to facts fixed outside the oracle itself.

Each test compares the oracle with a closed form, an invariant, a special case
that reduces to a textbook or library routine, a brute-force result on tiny
inputs, or a figure printed on the page -- never with a retyping of the
oracle's own formula.  Page cited: the iS-KV explainer ("iS-KV --
Basis-synchronized online low-rank KV compression -- What does it mean?").
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import (JointUnit, Oracle, Unit, bf16_round, brand_fold, drift, full_kv_bytes,
                    persistent_kv_bytes, rope)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent references (library routines, different formulations)
# ---------------------------------------------------------------------------

def rope_complex(x, pos, base=10000.0):
    """RoPE as complex multiplication: z_i = x_i + 1j*x_{i+d/2}, z_i * exp(1j*pos*f_i),
    with the usual inverse-frequency vector 1 / base**(arange(0, d, 2)/d)."""
    x = torch.as_tensor(np.asarray(x), dtype=torch.float64)
    d = x.shape[-1]
    inv = 1.0 / (base ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.as_tensor(np.asarray(pos), dtype=torch.float64)[..., None] * inv
    z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1).numpy()


def exact_attention(q, keys, vals, q_pos, scale, base=10000.0):
    """Uncompressed attention via torch's scaled_dot_product_attention (float64)."""
    L = keys.shape[0]
    kr = torch.as_tensor(rope_complex(keys, np.arange(L), base))
    qr = torch.as_tensor(rope_complex(q, np.full(q.shape[0], q_pos), base))
    out = torch.nn.functional.scaled_dot_product_attention(
        qr[None], kr[None], torch.as_tensor(np.asarray(vals))[None], scale=scale)
    return out[0].numpy()


def subspace_dist(B1, B2):
    """||P1 - P2||_2 for the projectors onto span(B1), span(B2)."""
    Q1, _ = np.linalg.qr(B1)
    Q2, _ = np.linalg.qr(B2)
    return float(np.linalg.norm(Q1 @ Q1.T - Q2 @ Q2.T, 2))


def lowrank(rng, L, d, k, noise=0.0):
    X = rng.standard_normal((L, k)) @ rng.standard_normal((k, d)) / math.sqrt(k)
    return X + noise * rng.standard_normal((L, d))


def run_unit(X, Y, d, r, window, storage="f64", block=64, sync=True, after_fold=None):
    u = Unit(d, r, window, X.shape[0] + block, storage, block)
    for t in range(X.shape[0]):
        u.append(X[t], Y[t])
        if u.ready:
            u.fold()
            if sync:
                u.sync()
            if after_fold:
                after_fold(u)
    return u


# ---------------------------------------------------------------------------
# bf16 storage rounding: pinned to torch's float32 -> bfloat16 conversion
# ---------------------------------------------------------------------------

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-39, -2.5e-40]]).astype(np.float32)
    # exact ties: values halfway between two bf16 numbers
    ties = (np.arange(1, 512, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -8) + 1
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# P7: RoPE invariants and the complex-multiplication form
# ---------------------------------------------------------------------------

def test_rope_matches_complex_form_and_invariants():
    rng = np.random.default_rng(1)
    d = 128
    x = rng.standard_normal((50, d))
    pos = rng.integers(0, 70000, 50)
    np.testing.assert_allclose(rope(x, pos), rope_complex(x, pos), rtol=0, atol=1e-10)
    np.testing.assert_allclose(np.linalg.norm(rope(x, pos), axis=1), np.linalg.norm(x, axis=1),
                               rtol=1e-13)
    np.testing.assert_array_equal(rope(x, np.zeros(50)), x)
    # scores depend only on the position difference
    q = rng.standard_normal(d)
    kp, qp, delta = rng.integers(0, 60000, 50), 61234, 1234
    s0 = rope(x, kp) @ rope(q, qp)
    s1 = rope(x, kp + delta) @ rope(q, qp + delta)
    np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-11 * np.abs(s0).max())


# ---------------------------------------------------------------------------
# P8: ring slots and no-fold decode = exact attention
# ---------------------------------------------------------------------------

def test_ring_slots_and_exact_attention_before_first_fold():
    rng = np.random.default_rng(2)
    d, r, W = 64, 8, 128
    L = W + 63                                   # one short of the first fold
    X, Y = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    u = run_unit(X, Y, d, r, W)
    assert u.n_c == 0 and not u.ready
    for p in range(L):
        np.testing.assert_array_equal(u.K.ring[p % (W + 64)], X[p])
        np.testing.assert_array_equal(u.V.ring[p % (W + 64)], Y[p])
    q = rng.standard_normal((3, d))
    scale = 1 / math.sqrt(d)
    np.testing.assert_allclose(u.decode(q, L - 1, scale), exact_attention(q, X, Y, L - 1, scale),
                               rtol=0, atol=1e-12)


def test_ring_slot_is_position_mod_window_plus_block():
    rng = np.random.default_rng(3)
    d, W = 16, 64
    X = rng.standard_normal((1000, d))
    u = run_unit(X, X, d, 4, W)
    for p in range(u.n_c, u.length):
        np.testing.assert_array_equal(u.K.ring[p % (W + 64)], X[p])
    assert u.length - u.n_c < W + 64 and u.length - u.n_c >= W


# ---------------------------------------------------------------------------
# P1: full rank (r = d) reproduces exact attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,W,L", [(32, 64, 600), (64, 128, 700)])
def test_full_rank_decode_is_exact_attention(d, W, L):
    rng = np.random.default_rng(4)
    X, Y = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    u = run_unit(X, Y, d, d, W)
    assert u.n_c >= 4 * 64
    q = rng.standard_normal((4, d))
    scale = 1 / math.sqrt(d)
    got = u.decode(q, L, scale)
    ref = exact_attention(q, X, Y, L, scale)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-11
    # every stored row is rebuilt exactly
    np.testing.assert_allclose(u.history("K"), X[: u.n_c], rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# P2: true rank <= r -> the incremental factorization is the batch SVD
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,r,k", [(128, 32, 24), (64, 64, 40), (128, 64, 64), (32, 8, 8)])
def test_rank_le_r_matches_batch_svd(d, r, k):
    rng = np.random.default_rng(5 + k)
    L = 64 * 12 + 64 + 17
    X = lowrank(rng, L, d, k)
    Y = lowrank(rng, L, d, k)
    u = run_unit(X, Y, d, r, 64)
    H = X[: u.n_c]
    rec = u.history("K")
    assert np.linalg.norm(rec - H) / np.linalg.norm(H) < 1e-11
    s_batch = np.linalg.svd(H, compute_uv=False)
    np.testing.assert_allclose(u.K.S[:k], s_batch[:k], rtol=1e-12, atol=1e-12 * s_batch[0])
    assert np.all(u.K.S[k:] <= 1e-9 * s_batch[0])
    _, _, vt = np.linalg.svd(H, full_matrices=False)
    assert subspace_dist(u.K.B[:, :k], vt[:k].T) < 1e-10
    # Independent route (incremental covariance, token by token): the top-k
    # eigenvectors of sum x^T x span the same subspace.
    G = np.zeros((d, d))
    for x in H:
        G += np.outer(x, x)
    w, V = np.linalg.eigh(G)
    assert subspace_dist(u.K.B[:, :k], V[:, ::-1][:, :k]) < 1e-9


def test_noisy_top_subspace_close_to_batch():
    """Sanity (not an exact pin): with rank-24 signal + 1% noise and r = 32,
    the gapped top-24 subspace agrees with the batch SVD's."""
    rng = np.random.default_rng(6)
    d, r, L = 128, 32, 64 * 30
    X = lowrank(rng, L, d, 24, noise=0.01)
    u = run_unit(X, X, d, r, 256)
    _, _, vt = np.linalg.svd(X[: u.n_c], full_matrices=False)
    assert subspace_dist(u.K.B[:, :24], vt[:24].T) < 1e-3


# ---------------------------------------------------------------------------
# P9: brute force on tiny inputs (d = 8, r = 2, block = 4)
# ---------------------------------------------------------------------------

def test_tiny_brute_force_block4():
    rng = np.random.default_rng(7)
    d, r, blk = 8, 2, 4
    X = lowrank(rng, 4 * 9 + 8 + 3, d, 2)
    u = run_unit(X, X, d, r, 8, block=blk)
    H = X[: u.n_c]
    U_, s, vt = np.linalg.svd(H)
    np.testing.assert_allclose(u.K.S, s[:2], rtol=1e-12)
    np.testing.assert_allclose(u.history("K"), H, rtol=0, atol=1e-12)
    # coefficients are the batch left singular vectors times sigma (up to sign)
    C = u.K.C[: u.n_c]
    for j in range(2):
        ref = U_[:, j] * s[j]
        sgn = np.sign(C[:, j] @ ref)
        np.testing.assert_allclose(C[:, j] * sgn, ref, rtol=0, atol=1e-11 * s[0])


# ---------------------------------------------------------------------------
# P3 / P4: orthonormal basis and Brand's coefficient invariant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["noisy", "rank5", "zeros", "full_rank", "rank5_r_eq_d"])
def test_basis_orthonormal_after_every_fold(kind):
    rng = np.random.default_rng(8)
    d, r = 64, 16
    L = 64 * 8 + 64
    if kind == "noisy":
        X = lowrank(rng, L, d, 24, noise=0.05)
    elif kind == "rank5":
        X = lowrank(rng, L, d, 5)
    elif kind == "zeros":
        X = np.zeros((L, d))
    elif kind == "rank5_r_eq_d":
        # fewer non-zero singular values than r: the null completion decides
        d = r = 32
        X = lowrank(rng, L, d, 5)
    else:
        r = d
        X = rng.standard_normal((L, d))
    errs = []
    run_unit(X, X, d, r, 64, after_fold=lambda u: errs.append(
        np.linalg.norm(u.K.B.T @ u.K.B - np.eye(r), 2)))
    assert len(errs) >= 8 and max(errs) < 1e-12


def test_coefficient_gram_is_diag_s_squared():
    rng = np.random.default_rng(9)
    d, r = 128, 32
    X = lowrank(rng, 64 * 10 + 64, d, 48, noise=0.02)
    u = run_unit(X, X, d, r, 64)
    C = u.K.C[: u.n_c]
    G = C.T @ C
    assert np.linalg.norm(G - np.diag(u.K.S ** 2)) / np.linalg.norm(G) < 1e-10


# ---------------------------------------------------------------------------
# P5: synchronization -- drift identities and ordering
# ---------------------------------------------------------------------------

def _drift_pair(X, d, r, W, folds_before):
    """(synchronized drift, basis-only drift, truncated-energy drift) of the next fold."""
    u = run_unit(X[: W + 64 * (folds_before + 1)], X[: W + 64 * (folds_before + 1)], d, r, W)
    n_old = u.n_c
    Ck, Bk = u.K.C[:n_old].copy(), u.K.B.copy()
    H0 = Ck @ Bk.T
    for t in range(u.length, u.length + 64):
        u.append(X[t], X[t])
    u.fold()
    Bn = u.K.B
    basis_only = drift(H0, Ck @ Bn.T)
    truncated = float(np.linalg.norm(H0 - H0 @ Bn @ Bn.T) / np.linalg.norm(H0))
    u.sync()
    synced = drift(H0, u.K.C[:n_old] @ Bn.T)
    return synced, basis_only, truncated


def test_sync_drift_zero_for_rank_le_r():
    rng = np.random.default_rng(10)
    X = lowrank(rng, 256 + 64 * 8, 128, 20)
    synced, basis_only, _ = _drift_pair(X, 128, 32, 256, 4)
    assert synced < 1e-12
    assert basis_only > 0.3


def test_sync_drift_equals_truncated_energy():
    rng = np.random.default_rng(11)
    X = lowrank(rng, 256 + 64 * 8, 128, 40, noise=0.05)
    synced, basis_only, truncated = _drift_pair(X, 128, 32, 256, 4)
    assert abs(synced - truncated) < 1e-12
    assert synced < 0.1 * basis_only


# ---------------------------------------------------------------------------
# P6: fused decode algebra ((p^T C) B^T for values, c B^T rebuilt keys)
# ---------------------------------------------------------------------------

def test_factored_value_route_equals_plain_decode():
    rng = np.random.default_rng(12)
    d, r, W = 64, 16, 64
    X, Y = lowrank(rng, 900, d, 16, 0.1), lowrank(rng, 900, d, 16, 0.1)
    u = run_unit(X, Y, d, r, W)
    q = rng.standard_normal((2, d))
    scale = 0.11
    n_c, L = u.n_c, u.length
    k_c = rope(u.K.C[:n_c] @ u.K.B.T, np.arange(n_c))
    k_w = rope(np.stack([u.K.ring[p % (W + 64)] for p in range(n_c, L)]), np.arange(n_c, L))
    s = np.concatenate([k_c, k_w]) @ rope(q, 1000).T * scale        # (L, g)
    p = np.exp(s - s.max(0))
    acc_c = p[:n_c].T @ u.V.C[:n_c]                                  # coefficient space
    acc_w = p[n_c:].T @ np.stack([u.V.ring[t % (W + 64)] for t in range(n_c, L)])
    fused = (acc_c @ u.V.B.T + acc_w) / p.sum(0)[:, None]
    np.testing.assert_allclose(u.decode(q, 1000, scale), fused, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# P10: grouped-query attention head map
# ---------------------------------------------------------------------------

def test_gqa_head_map_and_mha_special_case():
    rng = np.random.default_rng(13)
    B_, Hkv, Hq, d, r, W = 2, 2, 6, 32, 8, 64
    o = Oracle(B_, 1, Hkv, Hq, d, r, W, 600, storage="f64")
    k = rng.standard_normal((B_, 300, Hkv, d))
    v = rng.standard_normal((B_, 300, Hkv, d))
    for t in range(300):
        if o.append(0, k[:, t:t + 1], v[:, t:t + 1]):
            o.block_update(0)
            o.sync(0)
    q = rng.standard_normal((B_, Hq, d))
    out = o.decode_attn(0, q, 299)
    for b in range(B_):
        for h in range(Hq):
            u = o.unit(b, 0, h // 3)
            np.testing.assert_allclose(out[b, h], u.decode(q[b, h:h + 1], 299, o.scale)[0],
                                       rtol=0, atol=1e-14)
    # H_q = H_kv: multi-head attention; before any fold it is exact attention
    o2 = Oracle(1, 1, 3, 3, d, r, W, 200, storage="f64")
    k2, v2 = rng.standard_normal((1, 100, 3, d)), rng.standard_normal((1, 100, 3, d))
    o2.append(0, k2, v2)
    q2 = rng.standard_normal((1, 3, d))
    out2 = o2.decode_attn(0, q2, 99)
    for h in range(3):
        ref = exact_attention(q2[0, h:h + 1], k2[0, :, h], v2[0, :, h], 99, 1 / math.sqrt(d))
        np.testing.assert_allclose(out2[0, h:h + 1], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Storage rounding mode: ring rows and coefficients are bf16 values
# ---------------------------------------------------------------------------

def test_bf16_mode_stores_bf16_values():
    rng = np.random.default_rng(14)
    X = lowrank(rng, 400, 64, 8, 0.01)
    u = run_unit(X, X, 64, 16, 64, storage="bf16")
    for arr in (u.K.ring, u.K.C[: u.n_c], u.V.C[: u.n_c]):
        np.testing.assert_array_equal(bf16_round(arr), arr)


# ---------------------------------------------------------------------------
# Byte model, pinned to the page's figures
# ---------------------------------------------------------------------------

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    return rows


def test_full_kv_bytes_matches_page_figure():
    (tokens, layers, heads, d, eb, expect, gib), = _golden("full_kv_bytes.txt")
    got = full_kv_bytes(int(tokens), int(layers), int(heads), int(d), int(eb))
    assert got == int(expect)
    assert got / 2 ** 30 == float(gib)


def test_compression_ratio_is_inverse_budget():
    (ratio, budget, tol), = _golden("compression_ratio.txt")
    assert abs(1.0 / float(ratio) - float(budget)) < float(tol)


def test_persistent_bytes_full_rank_window_only():
    # with nothing compressed, the kept bytes are the exact rows plus the
    # (fixed) bases and singular values
    full = full_kv_bytes(300, 2, 4, 128, 2)
    kept = persistent_kv_bytes(0, 300, 2, 4, 128, 32, 2)
    assert kept - full == 2 * 4 * 2 * (128 * 32 * 4 + 32 * 4)


def test_persistent_bytes_counts_the_arrays_a_unit_keeps():
    """The byte model against a count of what an oracle unit actually stores
    after a stream (protected prefix, several folds, a ragged ring, r_V != r_K):
    coefficient rows that hold data, basis and singular-value entries, and the
    exact rows decode reads (positions written below P or at or after the
    compressed end).  Counted from the arrays and a log of the writes, not from
    the formula."""
    rng = np.random.default_rng(23)
    d, r, rv, window, P = 128, 16, 32, 64, 64
    L = P + 64 * 5 + 37
    u = Unit(d, r, window, L + 64, "bf16", prefix=P, r_v=rv)
    written = []
    for f in (u.K, u.V):
        orig = f.write

        def logged(pos, x, orig=orig, log=written):
            log.append(pos)
            orig(pos, x)
        f.write = logged
    for t in range(L):
        u.append(rng.standard_normal(d), rng.standard_normal(d))
        if u.ready:
            u.fold()
            u.sync()
    live = {p for p in written if p < P or p >= u.n_c}
    counted = 0
    for f, rf in ((u.K, r), (u.V, rv)):
        held = int(np.sum(np.any(f.C != 0.0, axis=1)))        # coefficient rows with data
        assert held == u.n_c - P and f.C.shape[1] == rf
        counted += held * rf * 2 + (f.B.size + f.S.size) * 4 + len(live) * d * 2
    assert counted == persistent_kv_bytes(u.n_c - P, len(live), 1, 1, d, r, 2, rank_v=rv)


# ---------------------------------------------------------------------------
# Brand step alone: the single-block special case is a truncated SVD
# ---------------------------------------------------------------------------

def test_first_fold_is_truncated_svd_of_block():
    rng = np.random.default_rng(15)
    d, r = 128, 32
    A = rng.standard_normal((64, d))
    B0, S0 = np.eye(d, r), np.zeros(r)
    Bn, Sn, M, C_blk = brand_fold(A, B0, S0)
    U_, s, vt = np.linalg.svd(A, full_matrices=False)
    np.testing.assert_allclose(Sn, s[:r], rtol=1e-12)
    assert subspace_dist(Bn, vt[:r].T) < 1e-10
    best = (U_[:, :r] * s[:r]) @ vt[:r]                 # Eckart-Young optimum
    np.testing.assert_allclose(C_blk @ Bn.T, best, rtol=0, atol=1e-11 * s[0])


# ---------------------------------------------------------------------------
# Protected prompt prefix: positions 0..P-1 stay exact and are never folded
# [iS-KV explainer, the window paragraph (paint-shop analogy): protected prompt
# positions stay exact; reading: a leading prefix of P positions]
# ---------------------------------------------------------------------------

def test_protected_prefix_exact_and_lossless_composition():
    """Full-rank random rows in the prefix, rank-12 noise-free rows after it,
    r = 16: the prefix must stay exact (compressing it would lose its full
    rank), the compressed part is lossless (rank <= r), so decode equals
    uncompressed attention over every position (torch SDPA, complex-form
    RoPE).  Compressing from position 0 instead of P, or a shifted position
    anywhere, fails this."""
    rng = np.random.default_rng(31)
    d, r, W, P = 64, 16, 64, 128
    L = P + 64 * 6 + 20
    X = np.vstack([rng.standard_normal((P, d)), lowrank(rng, L - P, d, 12)])
    Y = np.vstack([rng.standard_normal((P, d)), lowrank(rng, L - P, d, 12)])
    o = Oracle(1, 1, 1, 2, d, r, W, L + 64, storage="f64", prefix=P)
    u = o.unit(0, 0, 0)
    folds = 0
    for t in range(L):
        o.append(0, X[None, t:t + 1, None], Y[None, t:t + 1, None])
        if o.ready(0):
            o.block_update(0)
            o.sync(0)
            folds += 1
    assert folds >= 4 and u.compressed == 64 * folds and u.n_c == P + 64 * folds
    assert u.length - u.n_c >= W
    np.testing.assert_array_equal(u.K.prefix, X[:P])           # never touched by folds
    np.testing.assert_array_equal(u.V.prefix, Y[:P])
    np.testing.assert_allclose(u.history("K"), X[P:u.n_c], rtol=0, atol=1e-10)
    np.testing.assert_allclose(u.history("V"), Y[P:u.n_c], rtol=0, atol=1e-10)
    q = rng.standard_normal((1, 2, d))
    scale = 1 / math.sqrt(d)
    got = o.decode_attn(0, q, L + 3)[0]
    ref = exact_attention(q[0], X, Y, L + 3, scale)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-10


def test_prefix_longer_than_history_is_exact_attention_bf16():
    """P beyond the history: no fold ever happens and decode is uncompressed
    attention over the bf16-rounded rows (rounding by torch)."""
    rng = np.random.default_rng(32)
    d, r, W, P, L = 64, 16, 64, 256, 200
    # float32 inputs, as the library receives them (one rounding step to bf16)
    X = rng.standard_normal((L, d)).astype(np.float32).astype(np.float64)
    Y = rng.standard_normal((L, d)).astype(np.float32).astype(np.float64)
    u = Unit(d, r, W, 512, "bf16", 64, prefix=P)
    for t in range(L):
        u.append(X[t], Y[t])
        assert not u.ready
    assert u.compressed == 0
    to_bf16 = lambda a: torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    q = rng.standard_normal((3, d))
    got = u.decode(q, L - 1, 0.125)
    ref = exact_attention(q, to_bf16(X), to_bf16(Y), L - 1, 0.125)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-12


def test_prefix_must_be_block_multiple():
    with pytest.raises(ValueError):
        Unit(64, 16, 64, 512, "f64", 64, prefix=100)


# ---------------------------------------------------------------------------
# Separate K and V ranks [KV-CoRE page, Key Results: K and V are asymmetric]
# ---------------------------------------------------------------------------

def test_separate_v_rank_lossless_when_each_factor_fits():
    """K of rank 8 and V of rank 24 (both in span): with r_K = 16 and
    r_V = 32 every fold is lossless, so decode is exact attention; with
    r_V = r_K = 16 the V history is truncated and decode moves."""
    rng = np.random.default_rng(41)
    d, L, W = 64, 400, 64
    X = lowrank(rng, L, d, 8)
    Y = lowrank(rng, L, d, 24)
    q = rng.standard_normal((2, d))
    scale = 1 / math.sqrt(d)
    ref = exact_attention(q, X, Y, L + 1, scale)
    o = Oracle(1, 1, 1, 2, d, 16, W, L + 64, storage="f64", rank_v=32)
    u = o.unit(0, 0, 0)
    assert u.K.r == 16 and u.V.r == 32
    for t in range(L):
        u.append(X[t], Y[t])
        if u.ready:
            u.fold()
            u.sync()
    assert u.compressed >= 256
    got = u.decode(q, L + 1, scale)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-10
    # the V history is rebuilt exactly, the K history too
    np.testing.assert_allclose(u.history("V"), Y[: u.n_c], atol=1e-10)
    np.testing.assert_allclose(u.history("K"), X[: u.n_c], atol=1e-10)
    # same data with r_V = r_K: V is truncated (rank 24 > 16)
    v = run_unit(X, Y, d, 16, W)
    bad = v.decode(q, L + 1, scale)
    assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 1e-3


def test_separate_v_rank_leaves_k_factor_unchanged():
    """The K factor of a unit with r_V = 2 r_K is the K factor of the same
    stream with r_V = r_K: the factors never mix before decode."""
    rng = np.random.default_rng(42)
    d, L, W, r = 64, 330, 64, 16
    X = lowrank(rng, L, d, 30, 0.05)
    Y = lowrank(rng, L, d, 40, 0.05)
    a = run_unit(X, Y, d, r, W)
    b = Unit(d, r, W, L + 64, "f64", 64, r_v=2 * r)
    for t in range(L):
        b.append(X[t], Y[t])
        if b.ready:
            b.fold()
            b.sync()
    assert a.n_c == b.n_c
    np.testing.assert_array_equal(a.K.B, b.K.B)
    np.testing.assert_array_equal(a.K.C[: a.n_c], b.K.C[: b.n_c])
    assert b.V.B.shape == (d, 2 * r)
    # a wider V basis captures at least as much of the V history
    ea = np.linalg.norm(a.history("V") - Y[: a.n_c])
    eb = np.linalg.norm(b.history("V") - Y[: b.n_c])
    assert eb < ea


def test_persistent_bytes_with_separate_v_rank():
    """Closed form: per head, K keeps n_c*r_K coefficient elements, d*r_K + r_K
    fp32 basis/singular values and n_exact*d exact elements; V the same at r_V."""
    got = persistent_kv_bytes(1000, 300, 2, 4, 128, 32, 2, rank_v=64)
    k = 1000 * 32 * 2 + 128 * 32 * 4 + 32 * 4 + 300 * 128 * 2
    v = 1000 * 64 * 2 + 128 * 64 * 4 + 64 * 4 + 300 * 128 * 2
    assert got == 2 * 4 * (k + v)


# ---------------------------------------------------------------------------
# Deferred maintenance ["ASKV" design report, Design requirements: the new
# version is built aside and switched to later].  With 64 rows of ring slack,
# folding the ready block after k more appends gives exactly the state of a
# unit that folded on time and then took the same k appends: the fold reads
# only the block, B and S, none of which the later appends touch.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("storage,k", [("f32", 1), ("f32", 37), ("bf16", 64)])
def test_deferred_fold_commutes_with_later_appends(storage, k):
    rng = np.random.default_rng(55)
    d, r, W, T = 128, 16, 128, 64
    n = W + 2 * T + 64                        # two on-time folds, then the deferred one
    X = rng.standard_normal((n + k, 2, d)) @ np.diag(np.linspace(2, 0.1, d))
    on_time = Unit(d, r, W, 1024, storage)
    late = Unit(d, r, W, 1024, storage, slack=64)
    for p in range(n):
        for u in (on_time, late):
            u.append(X[p, 0], X[p, 1])
            if u.ready and p < n - 1:
                u.fold()
                u.sync()
    # the next block is ready (n - n_c = W + 64) in both; only on_time folds now
    assert on_time.ready and late.ready
    on_time.fold()
    on_time.sync()
    q = rng.standard_normal((4, d))
    for p in range(n, n + k):
        on_time.append(X[p, 0], X[p, 1])
        late.append(X[p, 0], X[p, 1])         # the ring slack holds them
    before = late.decode(q, n + k - 1, 1 / math.sqrt(d))
    late.fold()
    late.sync()
    assert late.n_c == on_time.n_c
    for a, b in ((late.K, on_time.K), (late.V, on_time.V)):
        np.testing.assert_array_equal(a.B, b.B)
        np.testing.assert_array_equal(a.S, b.S)
        np.testing.assert_array_equal(a.C[:late.n_c], b.C[:late.n_c])
    np.testing.assert_array_equal(late.decode(q, n + k - 1, 1 / math.sqrt(d)),
                                  on_time.decode(q, n + k - 1, 1 / math.sqrt(d)))
    # before the fold, the deferred unit is the pre-fold state: its block rows
    # are still exact, so its decode differs from the folded one by the
    # compression of that block (and the projection of the older history)
    assert np.abs(before - on_time.decode(q, n + k - 1, 1 / math.sqrt(d))).max() > 0
    # the slack is bounded: window + 128 rows past the compressed ones, no more
    full = Unit(d, r, W, 1024, storage, slack=64)
    for p in range(W + 128):
        full.append(X[p, 0], X[p, 1])
    with pytest.raises(RuntimeError):
        full.append(X[0, 0], X[0, 1])


# ---------------------------------------------------------------------------
# Bulk prefill [iS-KV explainer, the trade-off paragraph: prompts are
# compressed too]: folding a prompt's blocks with one deferred
# synchronization (suffix products of the M's) equals appending the tokens
# and folding + synchronizing each time the ring fills -- by associativity of
# the products, exactly in float64 storage.  A plausible mistake (a product
# in the wrong order, the wrong suffix for a block, the last block mapped)
# changes the history by O(1).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("prefix,n,hist", [(0, 640 + 37, 0), (64, 448, 0), (128, 128 + 64 * 3, 0)])
def test_bulk_prefill_equals_block_by_block(prefix, n, hist):
    rng = np.random.default_rng(71)
    d, r, W = 128, 16, 128
    X = rng.standard_normal((prefix + hist + n, 2, d)) @ np.diag(np.linspace(2, 0.05, d))
    a = Unit(d, r, W, 2048, "f64", prefix=prefix)
    b = Unit(d, r, W, 2048, "f64", prefix=prefix)
    # protected prefix and some history first (block by block in both)
    for p in range(prefix + hist):
        for u in (a, b):
            u.append(X[p, 0], X[p, 1])
            if u.ready:
                u.fold()
                u.sync()
    # a: the rest of the ring drains first when history was appended
    for u in (a, b):
        while u.length > u.n_c and u.length - u.n_c >= W + 64:
            u.fold()
            u.sync()
    if a.length != a.n_c:
        pytest.skip("ring not empty after the history")
    m = a.prefill(X[prefix + hist:, 0], X[prefix + hist:, 1])
    for p in range(prefix + hist, prefix + hist + n):
        b.append(X[p, 0], X[p, 1])
        if b.ready:
            b.fold()
            b.sync()
    assert m == (n - W) // 64 and a.n_c == b.n_c and a.length == b.length
    for fa, fb in ((a.K, b.K), (a.V, b.V)):
        np.testing.assert_allclose(fa.B, fb.B, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fa.C[:a.n_c], fb.C[:a.n_c], rtol=0,
                                   atol=1e-10 * np.abs(fb.C).max())
        live = [p % fa.slots for p in range(a.n_c, a.length)]     # slots of the exact rows
        np.testing.assert_array_equal(fa.ring[live], fb.ring[live])
    q = rng.standard_normal((4, d))
    np.testing.assert_allclose(a.decode(q, a.length - 1, 1 / math.sqrt(d)),
                               b.decode(q, b.length - 1, 1 / math.sqrt(d)), rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------
# Joint-head basis: one basis over a layer's KV heads [iS-KV explainer, the
# worked example and Table 1: ranks 64-128 compress 128-dim heads 4-7x]
# ---------------------------------------------------------------------------

def _joint_stream(rng, L, H, d, k):
    """K and V rows of H heads whose concatenation (H*d wide) has rank k:
    every head's rows are different mixtures of the same k latent factors."""
    Z = rng.standard_normal((L, k))
    X = (Z @ rng.standard_normal((k, H * d)) / math.sqrt(k)).reshape(L, H, d)
    Y = (rng.standard_normal((L, k)) @ rng.standard_normal((k, H * d)) / math.sqrt(k)).reshape(L, H, d)
    return X, Y


def _joint_exact(q, X, Y, q_pos, scale, g):
    """Per-head exact attention (torch SDPA): query rows h*g..(h+1)*g read head h."""
    H = X.shape[1]
    return np.concatenate([exact_attention(q[h * g:(h + 1) * g], X[:, h], Y[:, h], q_pos, scale)
                           for h in range(H)])


@pytest.mark.parametrize("H,d,r,k", [(4, 32, 16, 12), (2, 64, 32, 32), (3, 16, 48, 48)])
def test_joint_rank_le_r_is_exact_attention_per_head(H, d, r, k):
    """The heads' rows together have rank k <= r (r may exceed d, which a
    per-head basis cannot hold): every fold is lossless, the history is the
    stacked rows, S is the batch SVD of the (L x H*d) history, and decode of
    every KV head equals exact attention on that head's own rows."""
    rng = np.random.default_rng(61 + H)
    W, L, g = 64, 64 * 6 + 29, 2
    X, Y = _joint_stream(rng, L, H, d, k)
    u = JointUnit(H, d, r, W, L + 64, "f64")
    for t in range(L):
        u.append(X[t], Y[t])
        if u.ready:
            u.fold()
            u.sync()
    assert u.compressed >= 256 and u.K.B.shape == (H * d, r)
    Hk = X[: u.n_c].reshape(u.n_c, H * d)
    np.testing.assert_allclose(u.history("K"), Hk, atol=1e-10)
    s_batch = np.linalg.svd(Hk, compute_uv=False)
    np.testing.assert_allclose(u.K.S[:k], s_batch[:k], rtol=1e-11, atol=1e-11 * s_batch[0])
    q = rng.standard_normal((H * g, d))
    scale = 1 / math.sqrt(d)
    ref = _joint_exact(q, X, Y, L + 3, scale, g)
    got = u.decode(q, L + 3, scale)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-10
    # per-head bases sharing the same budget (rank r / H each) truncate
    # whenever a head's own rows (rank min(k, d)) exceed it
    if min(k, d) > r // H:
        per = [run_unit(X[:, h], Y[:, h], d, max(r // H, 1), W) for h in range(H)]
        bad = np.concatenate([per[h].decode(q[h * g:(h + 1) * g], L + 3, scale) for h in range(H)])
        assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 1e-4


def test_joint_full_rank_is_exact_attention():
    """r = H*d: the joint basis is square, every row is rebuilt exactly for
    arbitrary (full-rank) data, and decode is exact attention per head."""
    rng = np.random.default_rng(67)
    H, d, W, L, g = 2, 16, 64, 400, 3
    X = rng.standard_normal((L, H, d))
    Y = rng.standard_normal((L, H, d))
    u = JointUnit(H, d, H * d, W, L + 64, "f64")
    for t in range(L):
        u.append(X[t], Y[t])
        if u.ready:
            u.fold()
            u.sync()
    assert u.compressed >= 256
    q = rng.standard_normal((H * g, d))
    scale = 1 / math.sqrt(d)
    got = u.decode(q, L, scale)
    ref = _joint_exact(q, X, Y, L, scale, g)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-11


def test_joint_single_head_is_the_per_head_unit():
    """H = 1: the joint unit is the per-head unit, bit for bit (bf16 mode)."""
    rng = np.random.default_rng(71)
    d, r, W, L = 64, 16, 64, 300
    X, Y = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    j = JointUnit(1, d, r, W, L + 64, "bf16")
    u = Unit(d, r, W, L + 64, "bf16")
    for t in range(L):
        j.append(X[t][None], Y[t][None])
        u.append(X[t], Y[t])
        if u.ready:
            u.fold(); u.sync()
            j.fold(); j.sync()
    q = rng.standard_normal((4, d))
    np.testing.assert_array_equal(j.decode(q, L, 0.125), u.decode(q, L, 0.125))


def test_joint_oracle_layer_equals_joint_unit_and_gqa_map():
    """Oracle(joint_heads=True) drives one JointUnit per (sequence, layer);
    query head h reads KV head h // g, checked by permuting the KV heads'
    data: the outputs of the query-head groups permute with them."""
    rng = np.random.default_rng(73)
    B, H, Hq, d, r, W, n = 2, 4, 8, 32, 24, 64, 200
    o = Oracle(B, 1, H, Hq, d, r, W, n + 64, storage="f64", joint_heads=True)
    k = rng.standard_normal((B, n, H, d))
    v = rng.standard_normal((B, n, H, d))
    for t in range(n):
        if o.append(0, k[:, t:t + 1], v[:, t:t + 1]):
            o.block_update(0)
            o.sync(0)
    assert o.unit(0, 0, 0) is o.unit(0, 0, 3) and o.unit(0, 0, 0) is not o.unit(1, 0, 0)
    q = rng.standard_normal((B, Hq, d))
    out = o.decode_attn(0, q, n)
    for b in range(B):
        np.testing.assert_array_equal(out[b], o.unit(b, 0, 0).decode(q[b], n, o.scale))
    # permute the KV heads (and the query groups with them) in a fresh run
    perm = np.array([2, 0, 3, 1])
    qperm = q.reshape(B, H, Hq // H, d)[:, perm].reshape(B, Hq, d)
    o2 = Oracle(B, 1, H, Hq, d, r, W, n + 64, storage="f64", joint_heads=True)
    for t in range(n):
        if o2.append(0, k[:, t:t + 1, perm], v[:, t:t + 1, perm]):
            o2.block_update(0)
            o2.sync(0)
    out2 = o2.decode_attn(0, qperm, n)
    want = out.reshape(B, H, Hq // H, d)[:, perm].reshape(B, Hq, d)
    # a permutation of the row's columns leaves the SVD's spectrum and the
    # rebuilt rows unchanged up to rounding
    np.testing.assert_allclose(out2, want, rtol=0, atol=1e-9)


def test_joint_prefill_equals_block_by_block():
    """Bulk prefill of a joint unit (deferred sync by suffix products) equals
    folding and synchronizing block by block, in f64."""
    rng = np.random.default_rng(79)
    H, d, r, W, n = 2, 32, 16, 64, 64 * 5 + 40
    X = rng.standard_normal((n, H, d))
    Y = rng.standard_normal((n, H, d))
    a = JointUnit(H, d, r, W, n + 64, "f64")
    a.prefill(X, Y)
    b = JointUnit(H, d, r, W, n + 64, "f64")
    for t in range(n):
        b.append(X[t], Y[t])
        if b.ready:
            b.fold()
            b.sync()
    assert a.n_c == b.n_c and a.length == b.length
    np.testing.assert_allclose(a.history("K"), b.history("K"), atol=1e-10)
    q = rng.standard_normal((2 * H, d))
    np.testing.assert_allclose(a.decode(q, n, 0.2), b.decode(q, n, 0.2), atol=1e-10)


def test_joint_persistent_bytes_counts_the_arrays():
    """The joint byte model against a count of a joint unit's arrays after a
    stream: one coefficient row per token for all heads, one (H*d x r) basis
    per factor, and every head's exact rows."""
    rng = np.random.default_rng(83)
    H, d, r, rv, W = 8, 128, 64, 128, 64
    L = 64 * 4 + 21
    u = JointUnit(H, d, r, W, L + 64, "bf16", r_v=rv)
    for t in range(L):
        u.append(rng.standard_normal((H, d)), rng.standard_normal((H, d)))
        if u.ready:
            u.fold()
            u.sync()
    n_e = u.length - u.n_c
    counted = 0
    for f, rf in ((u.K, r), (u.V, rv)):
        held = int(np.sum(np.any(f.C != 0.0, axis=1)))
        assert held == u.n_c and f.C.shape[1] == rf and f.B.shape == (H * d, rf)
        counted += held * rf * 2 + (f.B.size + f.S.size) * 4 + n_e * H * d * 2
    assert counted == persistent_kv_bytes(u.n_c, n_e, 1, H, d, r, 2, rank_v=rv, joint_heads=True)
    # a joint basis at rank 64 keeps 1/8 of the per-head coefficient bytes at rank 64
    per_head = persistent_kv_bytes(u.n_c, 0, 1, H, d, 64, 2)
    joint = persistent_kv_bytes(u.n_c, 0, 1, H, d, 64, 2, joint_heads=True)
    assert joint < per_head
