"""Float64 CPU oracle for basis-synchronized online low-rank KV-cache compression.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this module imports nothing from the product path: the two
share no code, no tables and no constants.

What is computed, and where it comes from
-----------------------------------------
Page cited throughout: "iS-KV -- Basis-synchronized online low-rank KV
compression -- What does it mean?" (learnaivisually.com explainer of the iS-KV
paper), abbreviated [iS-KV explainer].

* Cache layout [iS-KV explainer, TL;DR and the window paragraph ("paint
  shop")]: the newest tokens are kept exact; every older position is kept as a
  short coefficient vector over a shared basis; nothing is evicted.
* Maintenance [iS-KV explainer, Jargon "Block-incremental SVD" and the drift
  paragraph]: each time 64 tokens leave the exact window they are folded into
  the factorization as one block with Brand's block-incremental SVD, solved on a
  core of (r+64) x (r+64) entries, so its cost is fixed as the history grows.
* Basis synchronization [iS-KV explainer, FAQ "What is basis synchronization?"
  and the drift paragraph]: when the basis changes, all stored coefficients are
  rewritten for the new basis in the same step.
* Keys are compressed before RoPE and RoPE is re-applied when a key is rebuilt
  [iS-KV explainer, Jargon "Pre-RoPE keys"].
* Attention at a new position runs over all of its predecessors, none dropped
  [iS-KV explainer, the re-attention paragraph].
* Persistent-KV bytes [iS-KV explainer, Jargon "Persistent-KV compression"].
* Protected prompt positions stay exact [iS-KV explainer, the window
  paragraph (the paint-shop analogy); the Jargon entry "Persistent-KV compression"
  counts them among the kept bytes].  Which positions, and how many, is not
  stated; the reading here is a leading prefix of P positions (P a multiple
  of 64, default 0) that is never folded: compression starts at position P.

* Deferred maintenance ["ASKV" design report, Design requirements:
  maintenance kept off the critical path, copy-on-write with a switch at a
  decode boundary].  With a slack of S extra ring rows, a block that is ready
  may be folded later: decode keeps attending over the pre-fold state (the
  block's rows still exact in the ring) while up to S more tokens arrive, and
  the fold, when applied, is the same Brand step on the same block, basis and
  singular values.  Default S = 0.

* A basis may span every KV head of a layer (JointUnit, Oracle(joint_heads=True)):
  ranks of 64-128 reach 4-7x compression of 128-dim heads [iS-KV explainer,
  the worked example and Table 1], which only a basis over several heads can
  give.  A token's row is then its heads' rows side by side, and the Brand
  fold, the sync and the coefficients are the same steps on those rows.

* K and V may take different ranks [KV-CoRE page, Key Results, the
  asymmetry of K and V: V needs more rank than K for the same energy].  The
  two factors never interact before decode, so a V factor of rank r_V is the
  same Brand fold and sync at a different r; the default is r_V = r.

Readings taken where the page is silent:
  window of W exact tokens plus up to 63 not yet folded (ring of W+64 rows,
  fold when it is full); basis per KV head, separate for K and V, rank r for
  both unless V is given its own rank r_V (see below);
  initial basis I[:, :r] with S = 0; core [[diag S, 0], [P, R_r^T]]; a
  rank-revealing residual basis and a unit-vector completion of null
  directions; half-split RoPE with base 10000 and fp64 angles; absolute
  positions from 0; scale 1/sqrt(d); bf16 round-to-nearest-even at every store
  in the "bf16" storage mode.

Decode is reached exactly (up to rounding order) by the fused route the GPU
takes, so here it is the plain definition: softmax attention over the rebuilt
cache.  The fold is an approximation built step by step, so it follows Brand's
update in order, with a LAPACK SVD of the core (numpy.linalg.svd).

Parity unpinned: the choice of directions with zero singular value (null
completion), the signs of singular vectors, exact ties between singular values,
and the page's printed drift and accuracy figures (they come from model
traces that are not available).
"""

from __future__ import annotations

import math

import numpy as np

EPS64 = float(np.finfo(np.float64).eps)
BLOCK = 64


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def bf16_round(x):
    """Round to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps the float32 exponent and 8 significant bits.  Rounding is
    done in one step from float64 (no intermediate float32).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    # bfloat16 subnormals share float32's smallest exponent (2**-126); below
    # it the spacing is fixed at 2**-133.
    e_eff = np.maximum(e, -125)
    scaled = np.ldexp(x, 8 - e_eff)           # 8 significant bits above the point
    return np.ldexp(np.rint(scaled), e_eff - 8)   # np.rint: ties to even


def store_round(x, storage: str):
    """Apply the rounding of one store in the given storage mode."""
    if storage == "bf16":
        return bf16_round(x)
    if storage == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if storage == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage mode {storage!r}")


# ----------------------------------------------------------------------------
# RoPE (half-split pairing), re-applied when a key is rebuilt
# [iS-KV explainer, Jargon "Pre-RoPE keys"]
# ----------------------------------------------------------------------------

def rope_theta(d: int, base: float) -> np.ndarray:
    """Frequencies theta_i = base**(-2i/d) for i < d/2, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope(x, pos, base: float = 10000.0):
    """Rotate feature pairs (i, i + d/2) of x by angle pos * theta_i.

    x has shape (..., d); pos broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ----------------------------------------------------------------------------
# Brand's block-incremental SVD step for one factor (K or V of one KV head)
# [iS-KV explainer, Jargon "Block-incremental SVD"; drift paragraph]
# ----------------------------------------------------------------------------

def _residual_basis(R, B, norm_a):
    """Orthonormal basis of the residual rows R, orthogonal to span(B).

    Rank-revealing: take the thin SVD of R^T and keep the left singular
    vectors whose singular value exceeds sqrt(eps) * ||A||_F; project them off
    B twice and re-orthonormalize.  Returns Q of shape (d, T) with the kept
    columns first and zero columns after them.
    """
    T, d = R.shape
    Q = np.zeros((d, T))
    if norm_a == 0.0:
        return Q
    w, sig, _ = np.linalg.svd(R.T, full_matrices=False)
    keep = sig > math.sqrt(EPS64) * norm_a
    qk = w[:, keep]
    for _ in range(2):
        qk = qk - B @ (B.T @ qk)
    if qk.shape[1]:
        qk, _ = np.linalg.qr(qk)
        Q[:, : qk.shape[1]] = qk
    return Q


def _complete_null_columns(Bn, sig_r, tol):
    """Replace columns whose singular value is <= tol by unit vectors.

    In column order, each such column becomes the e_k (k = lowest index among
    the largest) whose remainder after two Gram-Schmidt passes against the
    columns kept so far is largest, normalized.  Keeps the basis orthonormal
    when the core has fewer than r non-zero singular values.
    """
    d, r = Bn.shape
    bad = [j for j in range(r) if not sig_r[j] > tol]
    if not bad:
        return Bn
    Bn = Bn.copy()
    cols = [Bn[:, j] for j in range(r) if sig_r[j] > tol]
    for j in bad:
        basis = np.stack(cols, axis=1) if cols else np.zeros((d, 0))
        best_norm, best_vec = -1.0, None
        for k in range(d):
            e = np.zeros(d)
            e[k] = 1.0
            for _ in range(2):
                e = e - basis @ (basis.T @ e)
            nrm = float(np.linalg.norm(e))
            if nrm > best_norm:
                best_norm, best_vec = nrm, e
        Bn[:, j] = best_vec / best_norm
        cols.append(Bn[:, j])
    return Bn


def brand_fold(A, B, S):
    """Fold one block of rows A (T x d) into the rank-r factorization (B, S).

    State invariant (Brand): the stored coefficients C of the old rows satisfy
    C = U diag(S) with U orthonormal, so the old history is U diag(S) B^T.

    Steps:
      1. projection P = A B and residual R = A - P B^T, repeated once;
      2. residual basis Q (rank-revealing, orthogonal to B) and R_r^T = R Q;
      3. core K = [[diag S, 0], [P, R_r^T]] of size (r+T) x (r+T); the stacked
         history equals diag(U, I) K [B Q]^T, so K carries its singular values
         and right singular vectors;
      4. K = U' diag(s') V'^T by LAPACK, s' descending;
      5. keep r: B_new = [B Q] V'[:, :r] (null columns completed), S_new = s'[:r];
         M = B^T B_new rewrites old coefficients (basis synchronization);
         the block's own coefficients are P M + R_r^T (Q^T B_new).

    Returns (B_new, S_new, M, C_blk).
    """
    A = np.asarray(A, dtype=np.float64)
    T, d = A.shape
    r = B.shape[1]
    P = A @ B
    R = A - P @ B.T
    P2 = R @ B
    P = P + P2
    R = R - P2 @ B.T
    Q = _residual_basis(R, B, float(np.linalg.norm(A)))
    RrT = R @ Q                                        # (T, T)
    core = np.zeros((r + T, r + T))
    core[:r, :r] = np.diag(S)
    core[r:, :r] = P
    core[r:, r:] = RrT
    _, s, vt = np.linalg.svd(core)
    Vr = vt[:r].T                                      # (r+T, r)
    BQ = np.concatenate([B, Q], axis=1)                # (d, r+T)
    Bn = BQ @ Vr
    tol = BLOCK * (r + T) * EPS64 * float(s[0])
    Bn = _complete_null_columns(Bn, s[:r], tol)
    S_new = s[:r].copy()
    M = B.T @ Bn
    C_blk = P @ M + RrT @ (Q.T @ Bn)
    return Bn, S_new, M, C_blk


# ----------------------------------------------------------------------------
# One factor of one KV head: ring rows, basis, singular values, coefficients
# ----------------------------------------------------------------------------

class Factor:
    """K or V store of one (sequence, layer, KV head)."""

    def __init__(self, d: int, r: int, window: int, max_tokens: int, storage: str,
                 block: int = BLOCK, prefix: int = 0, slack: int = 0):
        if window % block:
            raise ValueError("window must be a multiple of the block size")
        if prefix % block or prefix < 0:
            raise ValueError("the protected prefix must be a multiple of the block size")
        self.d, self.r, self.window, self.block = d, r, window, block
        self.storage = storage
        self.slots = window + block + slack
        self.P = prefix
        self.prefix = np.zeros((prefix, d))   # exact rows of positions 0..P-1
        self.ring = np.zeros((self.slots, d))
        self.B = np.eye(d, r)                 # basis before the first block
        self.S = np.zeros(r)
        self.C = np.zeros((max_tokens, r))
        self.pending = None                    # M awaiting synchronization

    def write(self, pos: int, x):
        if pos < self.P:
            self.prefix[pos] = store_round(x, self.storage)
        else:
            self.ring[pos % self.slots] = store_round(x, self.storage)

    def block_rows(self, n_c: int):
        s0 = n_c % self.slots
        return self.ring[s0: s0 + self.block]

    def fold(self, n_c: int):
        Bn, Sn, M, C_blk = brand_fold(self.block_rows(n_c), self.B, self.S)
        self.C[n_c: n_c + self.block] = store_round(C_blk, self.storage)
        self.B, self.S, self.pending = Bn, Sn, M
        return M

    def sync(self, n_c_old: int):
        """Rewrite the old coefficients (positions P..n_c_old-1) for the
        current basis: C <- C M."""
        M = self.pending
        P = self.P
        self.C[P:n_c_old] = store_round(self.C[P:n_c_old] @ M, self.storage)
        self.pending = None

    def rebuilt(self, n_c: int, length: int):
        """Rows 0..length-1 as decode sees them: the exact protected prefix,
        C B^T of the compressed positions P..n_c-1, then exact ring rows."""
        out = np.empty((length, self.d))
        P = min(self.P, length)
        n_c = max(min(n_c, length), P)
        out[:P] = self.prefix[:P]
        out[P:n_c] = self.C[P:n_c] @ self.B.T
        for p in range(n_c, length):
            out[p] = self.ring[p % self.slots]
        return out


class Unit:
    """One (sequence, layer, KV head): a K factor, a V factor and counters."""

    def __init__(self, d, r, window, max_tokens, storage, block=BLOCK, prefix=0, r_v=None,
                 slack=0):
        self.K = Factor(d, r, window, max_tokens, storage, block, prefix, slack)
        self.V = Factor(d, r_v or r, window, max_tokens, storage, block, prefix, slack)
        self.slack = slack
        self.length = 0          # tokens appended (L)
        self.P = prefix          # protected exact prefix
        self.n_c = prefix        # end of the compressed positions P..n_c-1
        self.block = block
        self.window = window

    @property
    def compressed(self) -> int:
        """Tokens held as coefficients (N_c)."""
        return self.n_c - self.P

    @property
    def ready(self) -> bool:
        return self.length - self.n_c >= self.window + self.block

    def append(self, k, v):
        if self.length >= self.P and self.length - self.n_c >= self.window + self.block + self.slack:
            raise RuntimeError("ring full: fold the oldest block first")
        self.K.write(self.length, k)
        self.V.write(self.length, v)
        self.length += 1

    def fold(self):
        if not self.ready:
            raise RuntimeError("no block ready")
        mk = self.K.fold(self.n_c)
        mv = self.V.fold(self.n_c)
        self.n_c += self.block
        return mk, mv

    def sync(self):
        if self.K.pending is None:
            raise RuntimeError("no pending update")
        old = self.n_c - self.block
        self.K.sync(old)
        self.V.sync(old)

    def prefill(self, ks, vs):
        """Append prompt rows ks, vs (n x d) to a unit whose ring is empty,
        folding every block that leaves the window with its synchronization
        deferred: the blocks are folded in order exactly as appends would fold
        them, and afterwards each older row is multiplied once by the product
        of every M that came after it was written (the rows before the first
        block by M_0 ... M_{m-1}, block j's rows by M_{j+1} ... M_{m-1}).  Equal
        to folding and synchronizing block by block, by associativity, up to
        where the stores round.  Reading of the pages: the prompt is compressed
        like generated tokens [iS-KV explainer, the trade-off paragraph]; the
        single deferred synchronization is this library's restructuring."""
        ks = np.asarray(ks, dtype=np.float64)
        vs = np.asarray(vs, dtype=np.float64)
        if self.length != self.n_c or self.length < self.P:
            raise RuntimeError("prefill needs an empty ring")
        n = ks.shape[0]
        m = (n - self.window) // self.block if n >= self.window + self.block else 0
        n_c0 = self.n_c
        for f, xs in ((self.K, ks), (self.V, vs)):
            Ms = []
            for j in range(m):
                rows = store_round(xs[j * self.block:(j + 1) * self.block], f.storage)
                Bn, Sn, M, C_blk = brand_fold(rows, f.B, f.S)
                f.C[n_c0 + j * self.block: n_c0 + (j + 1) * self.block] = store_round(C_blk, f.storage)
                f.B, f.S = Bn, Sn
                Ms.append(M)
            if m:
                # suffix products S_j = M_j ... M_{m-1}
                suf = [None] * (m + 1)
                suf[m] = np.eye(f.r)
                for j in range(m - 1, -1, -1):
                    suf[j] = Ms[j] @ suf[j + 1]
                P = f.P
                f.C[P:n_c0] = store_round(f.C[P:n_c0] @ suf[0], f.storage)
                for j in range(m - 1):
                    a, b = n_c0 + j * self.block, n_c0 + (j + 1) * self.block
                    f.C[a:b] = store_round(f.C[a:b] @ suf[j + 1], f.storage)
        self.n_c = n_c0 + m * self.block
        for t in range(n):
            pos = self.length + t
            if pos >= self.n_c:
                self.K.write(pos, ks[t])
                self.V.write(pos, vs[t])
        self.length += n
        return m

    def decode(self, q, q_pos, scale, rope_base=10000.0):
        """Softmax attention of the query rows q (g x d) over every position.

        Keys: rebuilt (C_K B_K^T) or exact (ring), each rotated at its own
        position; queries rotated at q_pos; values rebuilt likewise, never
        rotated.
        """
        q = np.atleast_2d(np.asarray(q, dtype=np.float64))
        L = self.length
        keys = rope(self.K.rebuilt(self.n_c, L), np.arange(L), rope_base)
        vals = self.V.rebuilt(self.n_c, L)
        qr = rope(q, q_pos, rope_base)
        s = (qr @ keys.T) * scale                  # (g, L)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        return p @ vals

    def history(self, which: str):
        """Reconstructed pre-RoPE history C B^T of the compressed rows
        (positions P..n_c-1)."""
        f = self.K if which == "K" else self.V
        return f.C[self.P: self.n_c] @ f.B.T

    def load_state(self, length, n_c, ring_k, ring_v, Bk, Sk, Ck, Bv, Sv, Cv,
                   prefix_k=None, prefix_v=None):
        """Install a state (used to hand an oracle-made state to other code);
        n_c is the end position of the compressed rows."""
        self.length, self.n_c = int(length), int(n_c)
        for f, ring, B, S, C, pre in ((self.K, ring_k, Bk, Sk, Ck, prefix_k),
                                      (self.V, ring_v, Bv, Sv, Cv, prefix_v)):
            f.ring[:] = ring
            f.B = np.array(B, dtype=np.float64)
            f.S = np.array(S, dtype=np.float64)
            f.C[: n_c] = C[: n_c]
            if f.P:
                f.prefix[:] = pre
            f.pending = None


def drift(before, after):
    """Relative change of a reconstructed history caused by one update.

    Reading of [iS-KV explainer, drift paragraph]: drift is the change of the
    stored history from one update (not the error against the uncompressed
    cache); measured as ||H_after - H_before||_F / ||H_before||_F over the rows
    that existed before the update.
    """
    before = np.asarray(before, dtype=np.float64)
    after = np.asarray(after, dtype=np.float64)[: before.shape[0]]
    nb = np.linalg.norm(before)
    return float(np.linalg.norm(after - before) / nb) if nb > 0 else 0.0


class JointUnit(Unit):
    """One (sequence, layer) whose KV heads share one basis per factor.

    A token's row is its H heads' pre-RoPE rows side by side (H*d wide); the
    fold, the synchronization and the stored coefficient vector (rank r, one
    per token for all H heads) are Unit's on those rows.  Decode for KV head
    h rebuilds columns h*d..(h+1)*d of each row, rotates them at the row's
    position with d-dim RoPE and attends exactly as Unit does.

    Reading: the page reaches 4-7x compression at ranks 64-128 with 128-dim
    heads [iS-KV explainer, the worked example and Table 1], which a basis of
    one head cannot do at rank 128, so a basis must span several heads; the
    pages do not say which, and the group here is every KV head of a layer
    (Unit, one basis per head, is the other reading)."""

    def __init__(self, H, d, r, window, max_tokens, storage, block=BLOCK, prefix=0, r_v=None,
                 slack=0):
        super().__init__(H * d, r, window, max_tokens, storage, block, prefix, r_v, slack)
        self.H, self.hd = H, d

    def append(self, k, v):
        """k, v: (H, d) rows of the H KV heads at the next position."""
        super().append(np.asarray(k, dtype=np.float64).reshape(-1),
                       np.asarray(v, dtype=np.float64).reshape(-1))

    def prefill(self, ks, vs):
        """ks, vs: (n, H, d) prompt rows (see Unit.prefill)."""
        n = np.shape(ks)[0]
        return super().prefill(np.asarray(ks, dtype=np.float64).reshape(n, -1),
                               np.asarray(vs, dtype=np.float64).reshape(n, -1))

    def decode(self, q, q_pos, scale, rope_base=10000.0):
        """q: (H*g, d) query rows, g per KV head; rows h*g..(h+1)*g read KV head h."""
        q = np.atleast_2d(np.asarray(q, dtype=np.float64))
        g = q.shape[0] // self.H
        d, L = self.hd, self.length
        K = self.K.rebuilt(self.n_c, L)
        V = self.V.rebuilt(self.n_c, L)
        out = np.empty((q.shape[0], d))
        for h in range(self.H):
            keys = rope(K[:, h * d:(h + 1) * d], np.arange(L), rope_base)
            qr = rope(q[h * g:(h + 1) * g], q_pos, rope_base)
            s = (qr @ keys.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[h * g:(h + 1) * g] = p @ V[:, h * d:(h + 1) * d]
        return out


# ----------------------------------------------------------------------------
# Whole cache: batch x layers x KV heads, with grouped query heads
# ----------------------------------------------------------------------------

class Oracle:
    """The five verbs over every (sequence, layer, KV head), in float64.

    Shapes follow the library: k, v are [batch, n, kv_heads, d] (pre-RoPE),
    q is [batch, q_heads, d] (pre-RoPE), out is [batch, q_heads, d].  Query head
    h reads KV head h // (q_heads // kv_heads) (grouped-query attention).
    """

    def __init__(self, batch, num_layers, kv_heads, q_heads, head_dim, rank, window,
                 max_tokens, storage="bf16", rope_base=10000.0, softmax_scale=None,
                 block=BLOCK, prefix=0, rank_v=None, slack=0, joint_heads=False):
        if q_heads % kv_heads:
            raise ValueError("q_heads must be a multiple of kv_heads")
        self.batch, self.num_layers = batch, num_layers
        self.kv_heads, self.q_heads = kv_heads, q_heads
        self.d, self.r, self.window, self.block = head_dim, rank, window, block
        self.storage, self.rope_base = storage, rope_base
        self.scale = (1.0 / math.sqrt(head_dim)) if not softmax_scale else float(softmax_scale)
        self.prefix = prefix
        self.r_v = rank_v or rank
        self.joint = bool(joint_heads)
        if self.joint:
            # one JointUnit per (sequence, layer), listed once per KV head so
            # that unit(b, layer, h) and the per-head loops below still apply
            self.units = []
            for _ in range(batch):
                per_layer = []
                for _ in range(num_layers):
                    j = JointUnit(kv_heads, head_dim, rank, window, max_tokens, storage, block,
                                  prefix, self.r_v, slack)
                    per_layer.append([j] * kv_heads)
                self.units.append(per_layer)
        else:
            self.units = [[[Unit(head_dim, rank, window, max_tokens, storage, block, prefix,
                                 self.r_v, slack)
                            for _ in range(kv_heads)] for _ in range(num_layers)]
                          for _ in range(batch)]

    def unit(self, b, layer, h) -> Unit:
        return self.units[b][layer][h]

    def _heads(self):
        """KV heads that own a distinct unit (all, or only head 0 when joint)."""
        return range(1) if self.joint else range(self.kv_heads)

    def append(self, layer, k, v):
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        for b in range(self.batch):
            for t in range(k.shape[1]):
                if self.joint:
                    self.units[b][layer][0].append(k[b, t], v[b, t])
                    continue
                for h in range(self.kv_heads):
                    self.units[b][layer][h].append(k[b, t, h], v[b, t, h])
        return self.ready(layer)

    def ready(self, layer) -> bool:
        return self.units[0][layer][0].ready

    def block_update(self, layer):
        for b in range(self.batch):
            for h in self._heads():
                self.units[b][layer][h].fold()

    def sync(self, layer):
        for b in range(self.batch):
            for h in self._heads():
                self.units[b][layer][h].sync()

    def prefill(self, layer, k, v):
        """Unit.prefill for every (sequence, KV head) of the layer; k, v are
        [batch, n, kv_heads, d]."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        for b in range(self.batch):
            if self.joint:
                self.units[b][layer][0].prefill(k[b], v[b])
                continue
            for h in range(self.kv_heads):
                self.units[b][layer][h].prefill(k[b, :, h], v[b, :, h])

    def decode_attn(self, layer, q, q_pos):
        q = np.asarray(q, dtype=np.float64)
        g = self.q_heads // self.kv_heads
        out = np.zeros((self.batch, self.q_heads, self.d))
        for b in range(self.batch):
            if self.joint:
                out[b] = self.units[b][layer][0].decode(q[b], q_pos, self.scale, self.rope_base)
                continue
            for h in range(self.kv_heads):
                u = self.units[b][layer][h]
                out[b, h * g:(h + 1) * g] = u.decode(q[b, h * g:(h + 1) * g], q_pos,
                                                     self.scale, self.rope_base)
        return out


# ----------------------------------------------------------------------------
# Persistent-KV byte model [iS-KV explainer, Jargon "Persistent-KV compression"]
# ----------------------------------------------------------------------------

def full_kv_bytes(tokens, layers, kv_heads, head_dim, elem_bytes):
    """Bytes of an uncompressed K+V cache."""
    return 2 * tokens * layers * kv_heads * head_dim * elem_bytes


def persistent_kv_bytes(n_c, n_exact, layers, kv_heads, head_dim, rank, elem_bytes,
                        basis_bytes=4, rank_v=None, joint_heads=False):
    """Bytes kept between decode steps: coefficients, bases and singular values
    of K and V, plus the exact rows.  Model weights and temporary rebuild
    buffers are excluded.  rank_v (default rank) is the rank of the V factor.
    joint_heads: one basis (kv_heads*head_dim rows) and one coefficient row per
    token for all KV heads of a layer, instead of one per head."""
    if joint_heads:
        per_layer = sum(n_c * r * elem_bytes + kv_heads * head_dim * r * basis_bytes
                        + r * basis_bytes for r in (rank, rank_v or rank))
        return layers * (per_layer + 2 * kv_heads * n_exact * head_dim * elem_bytes)
    per_head = sum(n_c * r * elem_bytes + head_dim * r * basis_bytes + r * basis_bytes
                   + n_exact * head_dim * elem_bytes for r in (rank, rank_v or rank))
    return layers * kv_heads * per_head
