"""How far two correct implementations of the bf16-storage cache drift apart.

With bf16 storage every synchronization re-rounds every stored coefficient
(C <- bf16(C M)), and every fold rounds the new block's coefficients in the new
basis.  The basis itself is only defined up to rotations that leave the kept
subspace unchanged, and two implementations never compute it to the last bit:
a float32 implementation differs from the float64 oracle by rotations of the
order of the float32 rounding amplified by the singular-value gaps.  In exact
arithmetic (or with float32 storage) such a rotation changes nothing, because
C and B rotate together; with bf16 storage it changes which neighbouring bf16
value each re-rounded coefficient takes, and these differences accumulate
fold after fold like a random walk.

These tests run the float64 oracle against copies of itself whose fold is
perturbed in ways that leave it exact in real arithmetic:
  * the new basis rotated inside the kept subspace (B_new Z, M Z, C_blk Z with
    Z = expm(theta K), K a random skew matrix), theta = 1e-6 (the size of the
    rotation the GPU fold shows on identical states) and 1e-5 (a tenfold
    envelope);
  * the synchronization matrix M perturbed at float32 level (6e-8);
  * the whole fold evaluated in numpy float32.
They pin the reading that the attention-output tolerance (2e-3) applies to
identical imported states, while end-to-end bf16 runs are held to the envelope
below (WALK_ENVELOPE), which the GPU end-to-end tests use.  With float32
storage the same rotations leave the reconstruction unchanged (control).

Workload: the 32K GQA-layer generator (rank-32 signal + 1% noise, r = 32) at
2 KV heads / 8 query heads, window 128.
"""

import numpy as np
import pytest
import scipy.linalg

import oracle.iskv_oracle as O
import workloads

# End-to-end bf16 envelope (GPU vs oracle, same seeded stream): the largest
# divergence a per-fold rotation of 1e-5 produces below, times 1.25.
# keys: folds -> (history relative Frobenius error, attention output error)
WALK_ENVELOPE = {6: (3.0e-3, 7.5e-3), 20: (6.0e-3, 1.35e-2)}

W = workloads.with_(workloads.WORKLOADS[2], kv_heads=2, q_heads=8, window=128)
N_QUERIES = 4
ORIG_FOLD = O.brand_fold


def _rel(a, b):
    return float(np.max(np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)))


def _rotating(theta, seed):
    rng = np.random.default_rng(seed)

    def fold(A, B, S):
        Bn, Sn, M, C = ORIG_FOLD(A, B, S)
        r = Bn.shape[1]
        K = rng.standard_normal((r, r))
        Z = scipy.linalg.expm(theta * (K - K.T) / 2)
        return Bn @ Z, Sn, M @ Z, C @ Z
    return fold


def _perturb_m(rel, seed):
    rng = np.random.default_rng(seed)

    def fold(A, B, S):
        Bn, Sn, M, C = ORIG_FOLD(A, B, S)
        return Bn, Sn, M * (1.0 + rel * rng.standard_normal(M.shape)), C
    return fold


def _float32_fold():
    def fold(A, B, S):
        out = ORIG_FOLD(np.asarray(A, np.float32), np.asarray(B, np.float32), np.asarray(S, np.float32))
        return tuple(np.asarray(x, np.float64) for x in out)
    return fold


def _run(storage, fold, checkpoints):
    """Feed the stream, fold + sync whenever the ring fills; at each
    checkpoint (fold count) record the reconstructed histories and the
    attention outputs of N_QUERIES queries."""
    w = workloads.with_(W, storage=storage)
    L = 64 * max(checkpoints) + w.window + 21
    O.brand_fold = fold or ORIG_FOLD
    try:
        return _feed(w, L, checkpoints)
    finally:
        O.brand_fold = ORIG_FOLD


def _feed(w, L, checkpoints):
    ora = O.Oracle(w.batch, 1, w.kv_heads, w.q_heads, w.head_dim, w.rank, w.window, L + 64,
                   storage=w.storage)
    got, pos = {}, 0
    while pos < L:
        u = ora.unit(0, 0, 0)
        n = min(64, L - pos, w.window + 64 - (u.length - u.n_c))
        k, v = workloads.tokens(w, 0, pos, n)
        ora.append(0, k.astype(np.float32).astype(np.float64), v.astype(np.float32).astype(np.float64))
        pos += n
        if ora.ready(0):
            ora.block_update(0)
            ora.sync(0)
            nf = ora.unit(0, 0, 0).compressed // 64
            if nf in checkpoints:
                hist = [ora.unit(0, 0, h).history(x) for h in range(w.kv_heads) for x in "KV"]
                outs = [ora.decode_attn(0, workloads.query(w, 0, s).astype(np.float32).astype(np.float64),
                                        ora.unit(0, 0, 0).length - 1) for s in range(N_QUERIES)]
                got[nf] = (hist, outs)
    return got


def _divergence(a, b):
    """(history error, output error) per checkpoint of run b against run a."""
    res = {}
    for c in a:
        ha, oa = a[c]
        hb, ob = b[c]
        h = max(np.linalg.norm(x - y) / np.linalg.norm(y) for x, y in zip(hb, ha))
        o = max(_rel(x, y) for x, y in zip(ob, oa))
        res[c] = (h, o)
    return res


@pytest.fixture(scope="module")
def base_bf16():
    return _run("bf16", None, (6, 20))


def test_rotation_is_invisible_with_float32_storage():
    """Control: rotating the basis inside the kept subspace changes the
    reconstruction only at the float32 rounding of the stored values."""
    a = _run("f32", None, (6, 20))
    b = _run("f32", _rotating(1e-5, 5), (6, 20))
    for c, (h, o) in _divergence(a, b).items():
        assert h < 1e-6 and o < 1e-6, (c, h, o)


def test_bf16_rerounding_walk_at_gpu_rotation_size(base_bf16):
    """A 1e-6 rotation per fold already moves bf16 end-to-end outputs past the
    2e-3 output tolerance within 20 folds, and the history divergence grows
    with the fold count (re-rounding accumulates)."""
    d = _divergence(base_bf16, _run("bf16", _rotating(1e-6, 5), (6, 20)))
    (h6, o6), (h20, o20) = d[6], d[20]
    assert 5e-4 < h6 < h20 < 6e-3, d
    assert o20 > 2e-3, d


def test_bf16_walk_envelope(base_bf16):
    """The envelope the GPU end-to-end bf16 tests use is what a 1e-5 rotation
    per fold produces (two seeds), not an arbitrary loosening: the walk reaches
    at least 60% of it and stays below it."""
    worst = {c: [0.0, 0.0] for c in WALK_ENVELOPE}
    for seed in (5, 6):
        d = _divergence(base_bf16, _run("bf16", _rotating(1e-5, seed), (6, 20)))
        for c in WALK_ENVELOPE:
            worst[c][0] = max(worst[c][0], d[c][0])
            worst[c][1] = max(worst[c][1], d[c][1])
    for c, (hb, ob) in WALK_ENVELOPE.items():
        h, o = worst[c]
        assert 0.6 * hb <= h <= hb and 0.4 * ob <= o <= ob, (c, worst, WALK_ENVELOPE)


def test_bf16_walk_from_float32_level_perturbations(base_bf16):
    """Even perturbations at float32 level diverge with bf16 storage: M off by
    6e-8 relative, and the whole fold evaluated in numpy float32 (LAPACK)."""
    dm = _divergence(base_bf16, _run("bf16", _perturb_m(6e-8, 1), (6, 20)))
    df = _divergence(base_bf16, _run("bf16", _float32_fold(), (6, 20)))
    for d in (dm, df):
        assert d[20][0] > 3 * d[6][0] > 0, d         # grows with the fold count
        assert d[20][1] > 2e-4, d
    # the float32 fold stays inside the 1e-6 rotation's walk
    assert df[20][0] < 2.6e-3, df
