"""Thin ctypes binding of libmsgl (include/msgl.h).

Argument marshalling only: every function takes torch tensors, checks that
they are contiguous and on the device the call expects, passes their data
pointers and sizes to the C entry point of the same name, and raises
``MsglError`` on a non-OK status.  No computation happens here; there is no
CPU fallback.  If the library has not been built, importing raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsgl.so")

MSGL_OK = 0
MSGL_INVALID_ARG = 1
MSGL_UNSUPPORTED = 2
MSGL_WORKSPACE_TOO_SMALL = 3
MSGL_HIP_ERROR = 4

MSGL_F32 = 0
MSGL_BF16 = 1

# Every symbol include/msgl.h declares.
EXPORTS = (
    "msgl_last_error", "msgl_version", "msgl_store_kv", "msgl_rope_store_kv", "msgl_vocab_embed",
    "msgl_decode_workspace_bytes",
    "msgl_decode_attn", "msgl_decode_attn_noalloc", "msgl_noalloc_scratch_bytes", "msgl_prefill_attn",
    "msgl_decode_graph_create", "msgl_graph_launch", "msgl_graph_destroy", "msgl_validate_batch", "msgl_decode_shared_prefix_workspace_bytes",
    "msgl_decode_attn_shared_prefix", "msgl_validate_shared_prefix", "msgl_prefill_plan_bytes",
    "msgl_prefill_plan", "msgl_prefill_attn_planned", "msgl_check_batch",
)

# msgl_check_batch codes (include/msgl.h MSGL_CHECK_*)
CHECK_CODES = {"table_idx": 1, "seq_len": 2, "cached_len": 4, "cu_q": 8, "slot": 16, "page": 32,
               "out_loc": 64, "repeat": 128, "token_count": 256}


class MsglError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"msgl status {status}: {msg}")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run paged_kv_attention_slots_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    st = ctypes.c_int
    lib.msgl_last_error.restype = ctypes.c_char_p
    lib.msgl_last_error.argtypes = []
    lib.msgl_version.restype = ctypes.c_int
    lib.msgl_store_kv.restype = st
    lib.msgl_store_kv.argtypes = [P, P, I64, I32, I32, st, P, P, P, I32, P]
    lib.msgl_rope_store_kv.restype = st
    lib.msgl_rope_store_kv.argtypes = [P, P, P, P, I64, I32, I32, I32, st, P, P, P, P, I32,
                                       ctypes.c_double, P]
    lib.msgl_vocab_embed.restype = st
    lib.msgl_vocab_embed.argtypes = [P, P, I64, I64, I32, st, P, I32, P]
    lib.msgl_decode_workspace_bytes.restype = SZ
    lib.msgl_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.msgl_decode_attn.restype = st
    lib.msgl_decode_attn.argtypes = [P, P, P, P, P, I64, P, I32, P, P, I32, I32, I32, I32, I32, I32,
                                     I32, F, st, P, SZ, P]
    lib.msgl_decode_attn_noalloc.restype = st
    lib.msgl_decode_attn_noalloc.argtypes = [P, P, P, P, P, I64, P, I32, P, P, I32, I32, I32, I32, I32, I32,
                                             I32, F, st, P]
    lib.msgl_noalloc_scratch_bytes.restype = SZ
    lib.msgl_noalloc_scratch_bytes.argtypes = []
    lib.msgl_decode_shared_prefix_workspace_bytes.restype = SZ
    lib.msgl_decode_shared_prefix_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.msgl_decode_attn_shared_prefix.restype = st
    lib.msgl_decode_attn_shared_prefix.argtypes = [P, P, P, P, P, I64, P, I32, P, P, I32, P, P, I32, I32, I32,
                                                   I32, I32, I32, I32, I32, I32, F, st, P, SZ, P]
    lib.msgl_validate_shared_prefix.restype = st
    lib.msgl_validate_shared_prefix.argtypes = [P, I32, I32, P, P, I32, P, P, I32, I32, I32]
    lib.msgl_prefill_attn.restype = st
    lib.msgl_prefill_attn.argtypes = [P, P, P, P, P, I64, P, I32, P, P, P, P, I32, I32, I32, I32, I32,
                                      I32, I32, F, st, P]
    lib.msgl_prefill_plan_bytes.restype = SZ
    lib.msgl_prefill_plan_bytes.argtypes = [I32, I32, I32, I32]
    lib.msgl_prefill_plan.restype = st
    lib.msgl_prefill_plan.argtypes = [P, SZ, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, st]
    lib.msgl_prefill_attn_planned.restype = st
    lib.msgl_prefill_attn_planned.argtypes = [P, P, P, P, P, I64, P, I32, I32, I32, I32, I32, F, st, P, P, SZ,
                                              P]
    lib.msgl_decode_graph_create.restype = st
    lib.msgl_decode_graph_create.argtypes = [ctypes.POINTER(P), P, P, I64, P, P, P, P, P, P, P, I32, P,
                                             P, I32, I32, I32, I32, I32, I32, I32, F, st, P, SZ, P]
    lib.msgl_graph_launch.restype = st
    lib.msgl_graph_launch.argtypes = [P, P]
    lib.msgl_graph_destroy.restype = None
    lib.msgl_graph_destroy.argtypes = [P]
    lib.msgl_validate_batch.restype = st
    lib.msgl_validate_batch.argtypes = [P, I32, I32, P, P, P, P, I32, I32, I64, I32, P, I32, I64]
    lib.msgl_check_batch.restype = st
    lib.msgl_check_batch.argtypes = [P, I32, I32, P, P, P, P, I32, I32, I64, I32, P, I32, I64, P, P, P]
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != MSGL_OK:
        raise MsglError(status, lib.msgl_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSGL_F32
    if t.dtype == torch.bfloat16:
        return MSGL_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t: Optional[torch.Tensor], device: bool = True) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if device and not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return t.data_ptr()


def _i32(t: torch.Tensor) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise TypeError(f"index tensors are int32, got {t.dtype}")
    return t


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def msgl_version() -> int:
    return int(lib.msgl_version())


def msgl_last_error() -> str:
    return lib.msgl_last_error().decode()


def msgl_store_kv(k_pool, v_pool, k_new, v_new, out_loc, stream=None) -> None:
    S, G, d = k_pool.shape
    _check(lib.msgl_store_kv(_p(k_pool), _p(v_pool), S, G, d, _dt(k_pool), _p(k_new), _p(v_new),
                             _p(_i32(out_loc)), out_loc.numel(), _stream(stream)))


def msgl_rope_store_kv(q_out, q, k_pool, v_pool, k_new, v_new, positions, out_loc,
                       rope_base: float, stream=None) -> None:
    T, H, d = q.shape
    S, G, _ = k_pool.shape
    if q_out.shape != q.shape or k_new.shape != (T, G, d) or v_new.shape != (T, G, d):
        raise ValueError("q_out, k_new and v_new must match q [T, H, d] and the pools' [G, d]")
    if positions.numel() != T or out_loc.numel() != T:
        raise ValueError("positions and out_loc need one entry per token")
    _check(lib.msgl_rope_store_kv(_p(q_out), _p(q), _p(k_pool), _p(v_pool), S, H, G, d, _dt(k_pool),
                                  _p(k_new), _p(v_new), _p(_i32(positions)), _p(_i32(out_loc)), T,
                                  float(rope_base), _stream(stream)))


def msgl_vocab_embed(out, weight, ids, vocab_start: int = 0, stream=None) -> None:
    rows, hidden = weight.shape
    if out.shape != (ids.numel(), hidden) or out.dtype != weight.dtype:
        raise ValueError("out must be [num_tokens, hidden] in weight's dtype")
    _check(lib.msgl_vocab_embed(_p(out), _p(weight), int(vocab_start), rows, hidden, _dt(weight),
                                _p(_i32(ids)), ids.numel(), _stream(stream)))


def msgl_decode_workspace_bytes(batch: int, q_heads: int, head_dim: int, max_seq_len: int,
                                chunk: int = 0) -> int:
    return int(lib.msgl_decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, chunk))


def decode_workspace(batch: int, q_heads: int, head_dim: int, max_seq_len: int, chunk: int = 0,
                     device="cuda") -> torch.Tensor:
    """A workspace for msgl_decode_attn (zero-filled here; its contents need no initialisation)."""
    n = msgl_decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, chunk)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def msgl_decode_attn(out, lse, q, k_pool, v_pool, page_table, table_idx, seq_lens, max_seq_len: int,
                     workspace, page_size: int = 1, chunk: int = 0, sm_scale: Optional[float] = None,
                     stream=None) -> None:
    bs, H, d = q.shape
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    _check(lib.msgl_decode_attn(_p(out), _p(lse), _p(q), _p(k_pool), _p(v_pool), S,
                                _p(_i32(page_table)), page_table.shape[1], _p(_i32(table_idx)),
                                _p(_i32(seq_lens)), bs, H, G, d, page_size, max_seq_len, chunk,
                                sm_scale, _dt(q), _p(workspace), workspace.numel(), _stream(stream)))


def msgl_noalloc_scratch_bytes() -> int:
    return int(lib.msgl_noalloc_scratch_bytes())


def msgl_decode_attn_noalloc(out, lse, q, k_pool, v_pool, page_table, table_idx, seq_lens, max_seq_len: int,
                             page_size: int = 1, chunk: int = 0, sm_scale: Optional[float] = None,
                             stream=None) -> None:
    """msgl_decode_attn with the library's fixed scratch in place of a workspace."""
    bs, H, d = q.shape
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    _check(lib.msgl_decode_attn_noalloc(_p(out), _p(lse), _p(q), _p(k_pool), _p(v_pool), S,
                                        _p(_i32(page_table)), page_table.shape[1], _p(_i32(table_idx)),
                                        _p(_i32(seq_lens)), bs, H, G, d, page_size, max_seq_len, chunk,
                                        sm_scale, _dt(q), _stream(stream)))


def shared_prefix_workspace(batch: int, q_heads: int, head_dim: int, max_seq_len: int, chunk: int = 0,
                            device="cuda") -> torch.Tensor:
    """A workspace for msgl_decode_attn_shared_prefix (its contents need no initialisation)."""
    n = int(lib.msgl_decode_shared_prefix_workspace_bytes(batch, q_heads, head_dim, max_seq_len, chunk))
    return torch.empty(n, dtype=torch.uint8, device=device)


def msgl_decode_attn_shared_prefix(out, lse, q, k_pool, v_pool, page_table, table_idx, seq_lens, group_start,
                                   prefix_lens, max_group_size: int, max_prefix_len: int, max_seq_len: int,
                                   workspace, page_size: int = 1, chunk: int = 0,
                                   sm_scale: Optional[float] = None, stream=None) -> None:
    bs, H, d = q.shape
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    _check(lib.msgl_decode_attn_shared_prefix(
        _p(out), _p(lse), _p(q), _p(k_pool), _p(v_pool), S, _p(_i32(page_table)), page_table.shape[1],
        _p(_i32(table_idx)), _p(_i32(seq_lens)), bs, _p(_i32(group_start)), _p(_i32(prefix_lens)),
        group_start.numel() - 1, max_group_size, max_prefix_len, H, G, d, page_size, max_seq_len, chunk, sm_scale,
        _dt(q), _p(workspace), workspace.numel(), _stream(stream)))


def msgl_validate_shared_prefix(page_table, table_idx, seq_lens, group_start, prefix_lens, max_group_size: int,
                                max_prefix_len: int) -> None:
    """Check shared-prefix group metadata on host (CPU) tensors; raises MsglError."""
    c = lambda t: _p(_i32(t), device=False)
    _check(lib.msgl_validate_shared_prefix(c(page_table), page_table.shape[0], page_table.shape[1],
                                           c(table_idx), c(seq_lens), table_idx.numel(), c(group_start),
                                           c(prefix_lens), group_start.numel() - 1, max_group_size,
                                           max_prefix_len))


def msgl_prefill_attn(out, lse, q, k_pool, v_pool, page_table, table_idx, seq_lens, cached_lens, cu_q,
                      max_extend: int, page_size: int = 1, sm_scale: Optional[float] = None,
                      stream=None) -> None:
    T, H, d = q.shape
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    _check(lib.msgl_prefill_attn(_p(out), _p(lse), _p(q), _p(k_pool), _p(v_pool), S,
                                 _p(_i32(page_table)), page_table.shape[1], _p(_i32(table_idx)),
                                 _p(_i32(seq_lens)), _p(_i32(cached_lens)), _p(_i32(cu_q)),
                                 table_idx.numel(), T, max_extend, H, G, d, page_size, sm_scale,
                                 _dt(q), _stream(stream)))


def msgl_prefill_plan_bytes(batch: int, total_q: int, q_heads: int, kv_heads: int) -> int:
    return int(lib.msgl_prefill_plan_bytes(batch, total_q, q_heads, kv_heads))


def _host_i32(t) -> torch.Tensor:
    t = torch.as_tensor(t)
    if t.dtype != torch.int32:
        raise TypeError(f"index tensors are int32, got {t.dtype}")
    return t.cpu().contiguous()


def msgl_prefill_plan(seq_lens, cached_lens, cu_q, table_idx, rows: int, row_stride: int, q_heads: int,
                      kv_heads: int, head_dim: int = 128, dtype: int = MSGL_BF16) -> torch.Tensor:
    """Host plan of a prefill launch from host copies of the batch metadata.

    Returns the plan as a CPU int32 tensor (header, then one entry per query
    block, in launch order); copy it to the GPU for msgl_prefill_attn_planned.
    """
    sl, cl, cq, ti = (_host_i32(x) for x in (seq_lens, cached_lens, cu_q, table_idx))
    batch = ti.numel()
    total_q = int(cq[-1]) if cq.numel() else 0
    nbytes = msgl_prefill_plan_bytes(batch, total_q, q_heads, kv_heads)
    if nbytes == 0:
        raise MsglError(MSGL_INVALID_ARG, "invalid plan sizes")
    plan = torch.zeros(nbytes // 4, dtype=torch.int32)
    _check(lib.msgl_prefill_plan(_p(plan, device=False), nbytes, _p(sl, device=False), _p(cl, device=False),
                                 _p(cq, device=False), _p(ti, device=False), batch, total_q, rows, row_stride,
                                 q_heads, kv_heads, head_dim, dtype))
    return plan[: 8 + 8 * int(plan[3])].clone()


def msgl_prefill_attn_planned(out, lse, q, k_pool, v_pool, page_table, plan_host: torch.Tensor,
                              plan_dev: torch.Tensor, page_size: int = 1, sm_scale: Optional[float] = None,
                              stream=None) -> None:
    H, d = q.shape[1], q.shape[2]
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    if plan_dev.numel() < plan_host.numel():
        raise ValueError("the device plan is shorter than the host plan")
    _check(lib.msgl_prefill_attn_planned(_p(out), _p(lse), _p(q), _p(k_pool), _p(v_pool), S,
                                         _p(_i32(page_table)), page_table.shape[1], H, G, d, page_size,
                                         sm_scale, _dt(q), _p(_host_i32(plan_host), device=False),
                                         _p(_i32(plan_dev)), plan_host.numel() * 4, _stream(stream)))


class DecodeGraph:
    """Handle of a captured decode step (store_kv + decode attention)."""

    def __init__(self, handle: int, buffers: tuple):
        self._h = handle
        self._buffers = buffers  # the recorded tensors must outlive the graph

    def launch(self, stream=None) -> None:
        _check(lib.msgl_graph_launch(self._h, _stream(stream)))

    def destroy(self) -> None:
        if self._h:
            lib.msgl_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def msgl_decode_graph_create(k_pool, v_pool, k_new, v_new, out_loc, out, lse, q, page_table, table_idx,
                             seq_lens, max_seq_len: int, workspace, page_size: int = 1, chunk: int = 0,
                             sm_scale: Optional[float] = None, stream=None) -> DecodeGraph:
    bs, H, d = q.shape
    S, G, _ = k_pool.shape
    if sm_scale is None:
        sm_scale = d ** -0.5
    h = ctypes.c_void_p()
    _check(lib.msgl_decode_graph_create(
        ctypes.byref(h), _p(k_pool), _p(v_pool), S, _p(k_new), _p(v_new), _p(_i32(out_loc)), _p(out),
        _p(lse), _p(q), _p(_i32(page_table)), page_table.shape[1], _p(_i32(table_idx)),
        _p(_i32(seq_lens)), bs, H, G, d, page_size, max_seq_len, chunk, sm_scale, _dt(q),
        _p(workspace), workspace.numel(), _stream(stream)))
    return DecodeGraph(h.value, (k_pool, v_pool, k_new, v_new, out_loc, out, lse, q, page_table,
                                 table_idx, seq_lens, workspace))


def msgl_validate_batch(page_table, table_idx, seq_lens, cached_lens, cu_q, max_seq_len: int,
                        num_slots: int, page_size: int = 1, out_loc=None, dummy_slot: int = -1) -> None:
    """Check a batch's metadata on host (CPU) tensors; raises MsglError."""
    c = lambda t: None if t is None else _p(_i32(t), device=False)
    _check(lib.msgl_validate_batch(c(page_table), page_table.shape[0], page_table.shape[1],
                                   c(table_idx), c(seq_lens), c(cached_lens), c(cu_q),
                                   table_idx.numel(), max_seq_len, num_slots, page_size, c(out_loc),
                                   0 if out_loc is None else out_loc.numel(), dummy_slot))


def msgl_check_batch(page_table, table_idx, seq_lens, cached_lens, cu_q, max_seq_len: int, num_slots: int,
                     page_size: int = 1, out_loc=None, dummy_slot: int = -1, result=None, seen=None,
                     stream=None) -> torch.Tensor:
    """Enqueue the device-side metadata check on GPU tensors; returns the int32
    [4] result tensor (codes, flagged requests, first request, first token),
    valid once the stream reaches it.  seen: optional int32 scratch of
    ceil(num_slots / 32) words for the out_loc repeat check."""
    dev = page_table.device
    if result is None:
        result = torch.empty(4, dtype=torch.int32, device=dev)
    if seen is not None and seen.numel() < (num_slots + 31) // 32:
        raise ValueError("seen holds fewer than ceil(num_slots / 32) words")
    c = lambda t: None if t is None else _p(_i32(t))
    _check(lib.msgl_check_batch(c(page_table), page_table.shape[0], page_table.shape[1], c(table_idx),
                                c(seq_lens), c(cached_lens), c(cu_q), table_idx.numel(), max_seq_len, num_slots,
                                page_size, c(out_loc), 0 if out_loc is None else out_loc.numel(), dummy_slot,
                                c(result), c(seen), _stream(stream)))
    return result
