"""Python wrapper of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP path: it builds its own library with gcc, converts its own inputs,
and never calls into the product library.

The arithmetic lives in ``oracle.c``; this file only checks shapes, marshals
CPU tensors into the C calls, and composes the step the way the Mini-SGLang
Engine article orders a layer: write the new tokens' K/V into the pool first,
then attend over the page table.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_store_kv.argtypes = [P, P, I64, P, P, P, I64]
        lib.oracle_store_kv.restype = None
        lib.oracle_attention.argtypes = [ctypes.c_int, I64, P, P, P, P, I64, P, P, P,
                                         I64, I64, I64, ctypes.c_double, P, P]
        lib.oracle_attention.restype = None
        lib.oracle_rope.argtypes = [ctypes.c_int, P, I64, I64, I64, P, ctypes.c_double, P]
        lib.oracle_rope.restype = None
        lib.oracle_vocab_embed.argtypes = [P, I64, I64, I64, P, I64, P]
        lib.oracle_vocab_embed.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle supports fp32 and bf16 storage, got {t.dtype}")


def _cpu(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu").contiguous()


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def store_kv(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor,
             v_new: torch.Tensor, out_loc: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Pools after writing row t of ``k_new``/``v_new`` to slot ``out_loc[t]``.

    Returns new CPU tensors; the inputs are not modified."""
    kp, vp = _cpu(k_pool).clone(), _cpu(v_pool).clone()
    kn, vn = _cpu(k_new), _cpu(v_new)
    loc = _cpu(out_loc).to(torch.int32)
    assert kp.shape == vp.shape and kn.shape == vn.shape
    assert kp.dtype == kn.dtype and kp.shape[1:] == kn.shape[1:]
    assert loc.numel() == kn.shape[0]
    if loc.numel():
        assert int(loc.min()) >= 0 and int(loc.max()) < kp.shape[0]
    row_bytes = kp[0].numel() * kp.element_size()
    _load().oracle_store_kv(_ptr(kp), _ptr(vp), row_bytes, _ptr(kn), _ptr(vn), _ptr(loc),
                            loc.numel())
    return kp, vp


def attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
              page_table: torch.Tensor, table_idx: torch.Tensor, seq_lens: torch.Tensor,
              q_start: torch.Tensor, scale: Optional[float] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged causal GQA attention in fp64.

    ``q`` is ``[T, q_heads, head_dim]``; request b's queries are rows
    ``q_start[b] .. q_start[b+1]-1`` and sit at the last positions of its
    ``seq_lens[b]`` tokens.  Returns ``(out [T, H, d], lse [T, H])`` as float64."""
    q = _cpu(q)
    kp, vp = _cpu(k_pool), _cpu(v_pool)
    pt = _cpu(page_table).to(torch.int32)
    tix = _cpu(table_idx).to(torch.int32)
    sl = _cpu(seq_lens).to(torch.int32)
    qs = _cpu(q_start).to(torch.int32)
    T, H, d = q.shape
    G = kp.shape[1]
    n_req = tix.numel()
    assert kp.shape == vp.shape and kp.shape[2] == d and H % G == 0
    assert q.dtype == kp.dtype
    assert sl.numel() == n_req and qs.numel() == n_req + 1 and int(qs[-1]) == T
    assert pt.dim() == 2
    for b in range(n_req):
        n = int(qs[b + 1] - qs[b])
        L = int(sl[b])
        assert 1 <= n <= L <= pt.shape[1], (b, n, L)
        assert 0 <= int(tix[b]) < pt.shape[0]
        row = pt[int(tix[b]), :L]
        assert int(row.min()) >= 0 and int(row.max()) < kp.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty(T, H, d, dtype=torch.float64)
    lse = torch.empty(T, H, dtype=torch.float64)
    _load().oracle_attention(_dtype_code(q), n_req, _ptr(tix), _ptr(sl), _ptr(qs), _ptr(pt),
                             pt.shape[1], _ptr(q), _ptr(kp), _ptr(vp), H, G, d, float(scale),
                             _ptr(out), _ptr(lse))
    return out, lse


def rope(x: torch.Tensor, positions: torch.Tensor, base: float) -> torch.Tensor:
    """Rotary embedding of ``x`` ``[T, heads, head_dim]`` (fp32 or bf16) at
    ``positions`` ``[T]``, in fp64 (pairs i and i + head_dim/2 turn by
    ``positions[t] * base**(-2i/head_dim)``).  Returns a float64 tensor."""
    x = _cpu(x)
    pos = _cpu(positions).to(torch.int32)
    T, heads, d = x.shape
    assert d % 2 == 0 and pos.numel() == T and base > 0
    out = torch.empty(T, heads, d, dtype=torch.float64)
    _load().oracle_rope(_dtype_code(x), _ptr(x), T, heads, d, _ptr(pos), float(base), _ptr(out))
    return out


def rope_store_kv(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, v_pool: torch.Tensor,
                  positions: torch.Tensor, out_loc: torch.Tensor, base: float):
    """The layer's RoPE followed by the KV write: q and k turned by
    ``rope`` and, at slot ``out_loc[t]``, the K pool gets the turned k row and
    the V pool the v row.  Returns ``(q_rot, k_rot, v_pool')``: the turned
    rows in fp64 and the V pool after the write (the K pool's written rows are
    ``k_rot`` in the storage type, its other rows unchanged)."""
    q_rot = rope(q, positions, base)
    k_rot = rope(k_new, positions, base)
    _, vp = store_kv(v_pool, v_pool, k_new, v_new, out_loc)
    return q_rot, k_rot, vp


def vocab_embed(weight: torch.Tensor, ids: torch.Tensor, vocab_start: int = 0) -> torch.Tensor:
    """Embedding rows of ``ids`` from a vocabulary shard: ``weight`` ``[rows,
    hidden]`` holds the rows of ids ``vocab_start .. vocab_start + rows - 1``;
    other ids give zero rows.  Returns a new CPU tensor ``[T, hidden]`` in
    ``weight``'s dtype (rows copied bit for bit)."""
    wt = _cpu(weight)
    idx = _cpu(ids).to(torch.int32)
    assert wt.dim() == 2
    # poisoned, so that a row the C code left unwritten shows as NaN
    out = torch.full((idx.numel(), wt.shape[1]), float("nan"), dtype=wt.dtype)
    row_bytes = wt.shape[1] * wt.element_size()
    _load().oracle_vocab_embed(_ptr(wt), wt.shape[0], row_bytes, int(vocab_start), _ptr(idx),
                               idx.numel(), _ptr(out))
    return out


def step(w, scale: Optional[float] = None):
    """The whole step for a workload: store_kv, then attention of its new
    tokens.  Returns ``(k_pool', v_pool', out, lse)``."""
    kp, vp = store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    out, lse = attention(w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.cu_q, scale)
    return kp, vp, out, lse
