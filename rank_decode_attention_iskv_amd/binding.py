"""Thin ctypes binding of libiskv (include/iskv.h).

Argument marshalling only: every step of the compressed cache (append, fold,
synchronization, decode attention) runs in the HIP kernels of libiskv.so.
PyTorch is used for device memory (the workspace and caller tensors) and for
the stream handle.  There is no fallback: if libiskv.so is missing the import
fails loudly.

Functions keep the C names without the ``iskv_`` prefix; ``IskvCache`` owns a
workspace tensor and a context for convenience.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libiskv.so")

F32, BF16 = 0, 1
OK, EINVAL, ESTATE, ENOMEM, EDEVICE, ENUMERIC, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
FLAG_NONFINITE_CORE, FLAG_JACOBI_CAP, FLAG_NONFINITE_INPUT = 1, 2, 4


class Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32), ("window", ctypes.c_int32),
        ("block", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("storage", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("protected_prefix", ctypes.c_int32), ("rank_v", ctypes.c_int32),
        ("async_maintenance", ctypes.c_int32), ("joint_heads", ctypes.c_int32),
    ]


class Status(ctypes.Structure):
    _fields_ = [
        ("length", ctypes.c_int64), ("compressed", ctypes.c_int64),
        ("blocks_ready", ctypes.c_int32), ("pending_sync", ctypes.c_int32),
        ("folds", ctypes.c_int64), ("syncs", ctypes.c_int64),
        ("persistent_bytes", ctypes.c_uint64), ("full_bytes", ctypes.c_uint64),
        ("numeric_flags", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


EXPORTED = (
    "iskv_workspace_bytes", "iskv_state_bytes", "iskv_init", "iskv_append",
    "iskv_block_update", "iskv_sync", "iskv_discard_sync", "iskv_decode_attn",
    "iskv_append_decode", "iskv_status", "iskv_export_state", "iskv_import_state", "iskv_set_maintenance_stream",
    "iskv_join_maintenance", "iskv_destroy", "iskv_strerror",
    "iskv_append_ragged", "iskv_decode_attn_ragged", "iskv_seq_status",
    "iskv_decode_attn_noalloc", "iskv_noalloc_scratch_bytes",
    "iskv_maintain", "iskv_switch", "iskv_prefill", "iskv_prefill_layers",
)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libiskv.so not built at {path}; run "
                          "`python -m rank_decode_attention_iskv_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, SZ, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
    cfgp = ctypes.POINTER(Config)
    sig = {
        "iskv_workspace_bytes": (SZ, [cfgp]),
        "iskv_state_bytes": (SZ, [cfgp]),
        "iskv_init": (I, [cfgp, P, SZ, P, ctypes.POINTER(P)]),
        "iskv_append": (I, [P, I, P, P, I, I, ctypes.POINTER(I)]),
        "iskv_block_update": (I, [P, I]),
        "iskv_sync": (I, [P, I]),
        "iskv_discard_sync": (I, [P, I]),
        "iskv_decode_attn": (I, [P, I, P, I64, P]),
        "iskv_append_decode": (I, [P, I, P, P, I, P, I64, P, ctypes.POINTER(I)]),
        "iskv_status": (I, [P, I, ctypes.POINTER(Status)]),
        "iskv_export_state": (I, [P, I, P, SZ]),
        "iskv_import_state": (I, [P, I, P, SZ]),
        "iskv_set_maintenance_stream": (I, [P, P]),
        "iskv_join_maintenance": (I, [P, I]),
        "iskv_append_ragged": (I, [P, I, P, P, I, I, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(I)]),
        "iskv_decode_attn_ragged": (I, [P, I, P, ctypes.POINTER(I64), P]),
        "iskv_seq_status": (I, [P, I, I, ctypes.POINTER(Status)]),
        "iskv_decode_attn_noalloc": (I, [P, I, P, I64, P]),
        "iskv_noalloc_scratch_bytes": (SZ, [cfgp]),
        "iskv_maintain": (I, [P, I]),
        "iskv_switch": (I, [P, I, I]),
        "iskv_prefill": (I, [P, I, P, P, I, I]),
        "iskv_prefill_layers": (I, [P, I, ctypes.POINTER(I), ctypes.POINTER(P), ctypes.POINTER(P), I, I]),
        "iskv_destroy": (I, [P]),
        "iskv_strerror": (ctypes.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


class IskvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


def _check(code: int, what: str) -> int:
    if code != OK:
        raise IskvError(code, what)
    return code


def strerror(code: int) -> str:
    return lib().iskv_strerror(code).decode()


def make_config(batch, num_layers, num_kv_heads, num_q_heads, head_dim, rank, window,
                max_tokens, storage=BF16, rope_base=10000.0, softmax_scale=0.0, block=64,
                protected_prefix=0, rank_v=0, async_maintenance=0, joint_heads=0) -> Config:
    return Config(batch, num_layers, num_kv_heads, num_q_heads, head_dim, rank, window, block,
                  max_tokens, storage, rope_base, softmax_scale, protected_prefix, rank_v,
                  async_maintenance, joint_heads)


def ring_slots(cfg: Config) -> int:
    """Ring rows per unit: window + 64, and 64 more with copy-on-write maintenance."""
    return cfg.window + cfg.block * (2 if cfg.async_maintenance else 1)


def factor_ranks(cfg: Config):
    """(rank of K, rank of V); rank_v 0 means V shares the K rank."""
    return cfg.rank, (cfg.rank_v or cfg.rank)


def workspace_bytes(cfg: Config) -> int:
    return lib().iskv_workspace_bytes(ctypes.byref(cfg))


def state_bytes(cfg: Config) -> int:
    return lib().iskv_state_bytes(ctypes.byref(cfg))


def noalloc_scratch_bytes(cfg: Config) -> int:
    return lib().iskv_noalloc_scratch_bytes(ctypes.byref(cfg))


def _ptr(t) -> int:
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


class IskvCache:
    """A libiskv context plus the torch tensor that backs its workspace."""

    def __init__(self, cfg: Config, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.torch = torch
        n = workspace_bytes(cfg)
        if n == 0:
            raise IskvError(EINVAL, "iskv_workspace_bytes")
        # 256-byte alignment is guaranteed by the caching allocator
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        ctx = ctypes.c_void_p()
        _check(lib().iskv_init(ctypes.byref(cfg), ctypes.c_void_p(self.workspace.data_ptr()),
                               n, ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(ctx)),
               "iskv_init")
        self.ctx = ctx

    # -- verbs -------------------------------------------------------------
    def append(self, layer: int, k, v) -> bool:
        """k, v: device tensors [batch, n, kv_heads, head_dim], float32 or bfloat16."""
        torch = self.torch
        if k.dtype != v.dtype or k.shape != v.shape or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        dt = BF16 if k.dtype == torch.bfloat16 else F32
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k, v must be float32 or bfloat16")
        ready = ctypes.c_int(0)
        _check(lib().iskv_append(self.ctx, layer, ctypes.c_void_p(k.data_ptr()),
                                 ctypes.c_void_p(v.data_ptr()), int(k.shape[1]), dt,
                                 ctypes.byref(ready)), "iskv_append")
        return bool(ready.value)

    def block_update(self, layer: int = -1):
        _check(lib().iskv_block_update(self.ctx, layer), "iskv_block_update")

    def sync(self, layer: int = -1):
        _check(lib().iskv_sync(self.ctx, layer), "iskv_sync")

    def discard_sync(self, layer: int = -1):
        _check(lib().iskv_discard_sync(self.ctx, layer), "iskv_discard_sync")

    def decode_attn(self, layer: int, q, q_pos: int, out):
        """q, out: contiguous float32 device tensors [batch, q_heads, head_dim]."""
        torch = self.torch
        if q.dtype != torch.float32 or out.dtype != torch.float32:
            raise ValueError("q and out must be float32")
        if not q.is_contiguous() or not out.is_contiguous():
            raise ValueError("q and out must be contiguous")
        _check(lib().iskv_decode_attn(self.ctx, layer, ctypes.c_void_p(q.data_ptr()),
                                      int(q_pos), ctypes.c_void_p(out.data_ptr())),
               "iskv_decode_attn")
        return out

    def decode_attn_noalloc(self, layer: int, q, q_pos: int, out):
        """decode_attn with the split records in the library's static device
        array (allocates nothing)."""
        torch = self.torch
        if q.dtype != torch.float32 or out.dtype != torch.float32:
            raise ValueError("q and out must be float32")
        if not q.is_contiguous() or not out.is_contiguous():
            raise ValueError("q and out must be contiguous")
        _check(lib().iskv_decode_attn_noalloc(self.ctx, layer, ctypes.c_void_p(q.data_ptr()),
                                              int(q_pos), ctypes.c_void_p(out.data_ptr())),
               "iskv_decode_attn_noalloc")
        return out

    def append_decode(self, layer: int, k, v, q, q_pos: int, out) -> bool:
        """append(layer, k, v) of one token (k, v [batch, 1, kv_heads, head_dim])
        then decode_attn(layer, q, q_pos, out), in one launch.  Returns
        blocks_ready."""
        torch = self.torch
        if k.dtype != v.dtype or k.shape != v.shape or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        if k.dim() != 4 or k.shape[1] != 1:
            raise ValueError("k, v must be [batch, 1, kv_heads, head_dim]")
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k, v must be float32 or bfloat16")
        if q.dtype != torch.float32 or out.dtype != torch.float32:
            raise ValueError("q and out must be float32")
        if not q.is_contiguous() or not out.is_contiguous():
            raise ValueError("q and out must be contiguous")
        dt = BF16 if k.dtype == torch.bfloat16 else F32
        ready = ctypes.c_int(0)
        _check(lib().iskv_append_decode(self.ctx, layer, ctypes.c_void_p(k.data_ptr()),
                                        ctypes.c_void_p(v.data_ptr()), dt,
                                        ctypes.c_void_p(q.data_ptr()), int(q_pos),
                                        ctypes.c_void_p(out.data_ptr()), ctypes.byref(ready)),
               "iskv_append_decode")
        return bool(ready.value)

    def status(self, layer: int = 0, raise_numeric: bool = False) -> Status:
        st = Status()
        code = lib().iskv_status(self.ctx, layer, ctypes.byref(st))
        if code not in (OK, ENUMERIC) or (raise_numeric and code == ENUMERIC):
            raise IskvError(code, "iskv_status")
        return st

    def append_ragged(self, layer: int, k, v, counts) -> int:
        """Ragged append: k, v [batch, n, kv_heads, head_dim] device tensors;
        sequence b takes its first counts[b] rows.  Returns how many sequences
        have a full ring."""
        torch = self.torch
        if k.dtype != v.dtype or k.shape != v.shape or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k, v must be float32 or bfloat16")
        if len(counts) != self.cfg.batch:
            raise ValueError("one count per sequence")
        dt = BF16 if k.dtype == torch.bfloat16 else F32
        cnt = (ctypes.c_int32 * len(counts))(*[int(x) for x in counts])
        ready = ctypes.c_int(0)
        _check(lib().iskv_append_ragged(self.ctx, layer, ctypes.c_void_p(k.data_ptr()),
                                        ctypes.c_void_p(v.data_ptr()), int(k.shape[1]), dt, cnt,
                                        ctypes.byref(ready)), "iskv_append_ragged")
        return ready.value

    def decode_attn_ragged(self, layer: int, q, q_pos, out):
        """decode_attn with one query position per sequence (q_pos: [batch])."""
        torch = self.torch
        if q.dtype != torch.float32 or out.dtype != torch.float32:
            raise ValueError("q and out must be float32")
        if not q.is_contiguous() or not out.is_contiguous():
            raise ValueError("q and out must be contiguous")
        if len(q_pos) != self.cfg.batch:
            raise ValueError("one query position per sequence")
        qp = (ctypes.c_int64 * len(q_pos))(*[int(x) for x in q_pos])
        _check(lib().iskv_decode_attn_ragged(self.ctx, layer, ctypes.c_void_p(q.data_ptr()), qp,
                                             ctypes.c_void_p(out.data_ptr())),
               "iskv_decode_attn_ragged")
        return out

    def seq_status(self, layer: int, seq: int) -> Status:
        st = Status()
        code = lib().iskv_seq_status(self.ctx, layer, seq, ctypes.byref(st))
        if code not in (OK, ENUMERIC):
            raise IskvError(code, "iskv_seq_status")
        return st

    def export_state(self, layer: int) -> bytearray:
        n = state_bytes(self.cfg)
        buf = bytearray(n)
        c_buf = (ctypes.c_char * n).from_buffer(buf)
        _check(lib().iskv_export_state(self.ctx, layer, c_buf, n), "iskv_export_state")
        return buf

    def import_state(self, layer: int, blob) -> None:
        n = state_bytes(self.cfg)
        if len(blob) < n:
            raise ValueError("state blob too small")
        buf = blob if isinstance(blob, bytearray) else bytearray(blob)
        c_buf = (ctypes.c_char * len(buf)).from_buffer(buf)
        _check(lib().iskv_import_state(self.ctx, layer, c_buf, len(buf)), "iskv_import_state")

    def set_maintenance_stream(self, stream) -> None:
        """Run block updates and syncs on `stream` (a torch.cuda.Stream), off the
        init stream; None returns to single-stream operation."""
        self.mstream = stream                     # kept alive with the cache
        ptr = ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)
        _check(lib().iskv_set_maintenance_stream(self.ctx, ptr), "iskv_set_maintenance_stream")

    def join_maintenance(self, layer: int = -1) -> None:
        _check(lib().iskv_join_maintenance(self.ctx, layer), "iskv_join_maintenance")

    def prefill(self, layer: int, k, v) -> None:
        """Prompt tokens k, v (device tensors [batch, n, kv_heads, head_dim],
        float32 or bfloat16) appended to a layer with an empty ring, every
        block that leaves the window folded in one pass (iskv_prefill)."""
        torch = self.torch
        if k.dtype != v.dtype or k.shape != v.shape or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        if k.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k, v must be float32 or bfloat16")
        dt = BF16 if k.dtype == torch.bfloat16 else F32
        _check(lib().iskv_prefill(self.ctx, layer, ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), int(k.shape[1]), dt), "iskv_prefill")

    def prefill_layers(self, layers, ks, vs) -> None:
        """iskv_prefill_layers: one input (k, v device tensors [batch, n, kv_heads,
        head_dim], all of one shape and dtype) per layer."""
        torch = self.torch
        n = len(layers)
        if not (len(ks) == len(vs) == n) or n == 0:
            raise ValueError("one k and one v per layer")
        for k, v in zip(ks, vs):
            if k.dtype != ks[0].dtype or k.shape != ks[0].shape or v.shape != k.shape or \
                    v.dtype != k.dtype or not k.is_contiguous() or not v.is_contiguous():
                raise ValueError("k and v must be contiguous tensors of one shape and dtype")
        if ks[0].dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k, v must be float32 or bfloat16")
        dt = BF16 if ks[0].dtype == torch.bfloat16 else F32
        la = (ctypes.c_int * n)(*layers)
        kp = (ctypes.c_void_p * n)(*[k.data_ptr() for k in ks])
        vp = (ctypes.c_void_p * n)(*[v.data_ptr() for v in vs])
        _check(lib().iskv_prefill_layers(self.ctx, n, la, kp, vp, int(ks[0].shape[1]), dt),
               "iskv_prefill_layers")

    def maintain(self, layer: int = -1) -> None:
        """Copy-on-write maintenance (async_maintenance contexts): enqueue the
        fold + sync of the layer into its other generation and return."""
        _check(lib().iskv_maintain(self.ctx, layer), "iskv_maintain")

    def switch(self, layer: int, wait: bool = False) -> bool:
        """Switch the layer to its new generation if its maintenance finished
        (wait: order the init stream after it).  True if it switched."""
        r = lib().iskv_switch(self.ctx, layer, 1 if wait else 0)
        if r < 0:
            _check(r, "iskv_switch")
        return r == 1

    def destroy(self):
        if getattr(self, "ctx", None):
            lib().iskv_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# -- state blob helpers (layout documented at iskv_state_bytes) --------------

def unpack_state(cfg: Config, blob):
    """Split a state blob into numpy arrays per (unit, K|V); n_c is the
    compressed token count (rows protected_prefix .. protected_prefix+n_c-1)."""
    import numpy as np
    d, T, S = cfg.head_dim, cfg.max_tokens, ring_slots(cfg)
    ranks = factor_ranks(cfg)
    Pp = cfg.protected_prefix
    length, n_c = np.frombuffer(bytes(blob[:16]), dtype=np.int64)
    f = np.frombuffer(bytes(blob[16:]), dtype=np.float32)
    units = cfg.batch * cfg.num_kv_heads
    out = []
    o = 0
    for u in range(units):
        xs = []
        for x in range(2):
            r = ranks[x]
            B = f[o: o + d * r].reshape(d, r); o += d * r
            Sv = f[o: o + r]; o += r
            C = f[o: o + T * r].reshape(T, r); o += T * r
            ring = f[o: o + S * d].reshape(S, d); o += S * d
            prefix = f[o: o + Pp * d].reshape(Pp, d); o += Pp * d
            xs.append(dict(basis=B, S=Sv, coef=C, ring=ring, prefix=prefix))
        out.append(xs)
    return int(length), int(n_c), out


def pack_state(cfg: Config, length: int, n_c: int, units) -> bytearray:
    """Inverse of unpack_state; units (any iterable, consumed once, one entry
    per unit in order) gives units[u][x] with basis, S, coef (rows by
    position), ring and, with a protected prefix, prefix arrays.  The blob is
    filled in place, so a generator of units never holds more than one unit."""
    import numpy as np
    d, T, S = cfg.head_dim, cfg.max_tokens, ring_slots(cfg)
    ranks = factor_ranks(cfg)
    Pp = cfg.protected_prefix
    blob = bytearray(state_bytes(cfg))
    np.frombuffer(blob, dtype=np.int64, count=2)[:] = (length, n_c)
    f = np.frombuffer(blob, dtype=np.float32, offset=16)
    o = 0
    for xs in units:
        for r, x in zip(ranks, xs):
            f[o: o + d * r] = np.asarray(x["basis"], np.float32).reshape(d * r); o += d * r
            f[o: o + r] = np.asarray(x["S"], np.float32).reshape(r); o += r
            C = np.asarray(x["coef"], np.float32)[:T]
            f[o: o + C.size] = C.reshape(-1)
            f[o + C.size: o + T * r] = 0.0
            o += T * r
            f[o: o + S * d] = np.asarray(x["ring"], np.float32).reshape(S * d); o += S * d
            if Pp:
                f[o: o + Pp * d] = np.asarray(x["prefix"], np.float32).reshape(Pp * d); o += Pp * d
    if o != f.size:
        raise ValueError("state blob: wrong number of units")
    return blob
