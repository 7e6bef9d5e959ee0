"""Drive one attention step of a workload through the C ABI.

Plumbing only: allocate outputs and workspaces with torch on the workload's
device and call the binding.  All computation happens in libmsgl's kernels.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib
from .workloads import Workload


@dataclasses.dataclass
class StepResult:
    out: torch.Tensor
    lse: Optional[torch.Tensor]
    k_pool: torch.Tensor
    v_pool: torch.Tensor


def store_kv(w: Workload, k_pool: torch.Tensor, v_pool: torch.Tensor, stream=None) -> None:
    _lib.msgl_store_kv(k_pool, v_pool, w.k_new, w.v_new, w.out_loc, stream=stream)


def decode_attn(w: Workload, k_pool, v_pool, out=None, lse=None, workspace=None, chunk: int = 0,
                with_lse: bool = True, stream=None):
    dev = w.q.device
    if out is None:
        out = torch.empty_like(w.q)
    if lse is None and with_lse:
        lse = torch.empty(w.bs, w.q_heads, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _lib.decode_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, chunk, device=dev)
    _lib.msgl_decode_attn(out, lse, w.q, k_pool, v_pool, w.page_table, w.table_idx, w.seq_lens,
                          w.max_seq_len, workspace, page_size=w.page_size, chunk=chunk,
                          sm_scale=w.sm_scale, stream=stream)
    return out, lse


def prefill_attn(w: Workload, k_pool, v_pool, out=None, lse=None, with_lse: bool = True, stream=None):
    dev = w.q.device
    if out is None:
        out = torch.empty_like(w.q)
    if lse is None and with_lse:
        lse = torch.empty(w.num_tokens, w.q_heads, dtype=torch.float32, device=dev)
    max_extend = int((w.seq_lens - w.cached_lens).max().item())
    _lib.msgl_prefill_attn(out, lse, w.q, k_pool, v_pool, w.page_table, w.table_idx, w.seq_lens,
                           w.cached_lens, w.cu_q, max_extend, page_size=w.page_size,
                           sm_scale=w.sm_scale, stream=stream)
    return out, lse


def prefill_plan(w: Workload):
    """The host plan of w's prefill launch: (host int32 tensor, its device copy)."""
    plan = _lib.msgl_prefill_plan(w.seq_lens.cpu(), w.cached_lens.cpu(), w.cu_q.cpu(), w.table_idx.cpu(),
                                  w.page_table.shape[0], w.page_table.shape[1], w.q_heads, w.kv_heads,
                                  w.head_dim, _lib._dt(w.q))
    return plan, plan.to(w.q.device)


def prefill_attn_planned(w: Workload, k_pool, v_pool, plan=None, out=None, lse=None, with_lse: bool = True,
                         stream=None):
    dev = w.q.device
    if plan is None:
        plan = prefill_plan(w)
    if out is None:
        out = torch.empty_like(w.q)
    if lse is None and with_lse:
        lse = torch.empty(w.num_tokens, w.q_heads, dtype=torch.float32, device=dev)
    _lib.msgl_prefill_attn_planned(out, lse, w.q, k_pool, v_pool, w.page_table, plan[0], plan[1],
                                   page_size=w.page_size, sm_scale=w.sm_scale, stream=stream)
    return out, lse


def run_step(w: Workload, chunk: int = 0, with_lse: bool = True, in_place: bool = False) -> StepResult:
    """store_kv then attention (decode or prefill by the workload's mode)."""
    kp = w.k_pool if in_place else w.k_pool.clone()
    vp = w.v_pool if in_place else w.v_pool.clone()
    store_kv(w, kp, vp)
    if w.mode == "decode":
        out, lse = decode_attn(w, kp, vp, chunk=chunk, with_lse=with_lse)
    else:
        out, lse = prefill_attn(w, kp, vp, with_lse=with_lse)
    return StepResult(out, lse, kp, vp)


def rope_store_kv(w: Workload, k_pool, v_pool, rope_base: float, q_out=None, stream=None):
    """The layer's RoPE fused with the KV write: returns the rotated q (a new
    tensor unless ``q_out`` is given; ``q_out=w.q`` rotates in place); the
    rotated k rows and the v rows land in the pools at ``w.out_loc``."""
    if q_out is None:
        q_out = torch.empty_like(w.q)
    _lib.msgl_rope_store_kv(q_out, w.q, k_pool, v_pool, w.k_new, w.v_new, w.positions, w.out_loc,
                            rope_base, stream=stream)
    return q_out
