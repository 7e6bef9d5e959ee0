"""Shared helpers of the GPU parity tests (comparison and sampling only)."""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np
import torch

BF16_TOL = 2e-2
F32_TOL = 1e-5
ROWSUM_TOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)


def tol(w) -> float:
    return F32_TOL if w.dtype == torch.float32 else BF16_TOL


def store_mismatch(w, kp_gpu: torch.Tensor, vp_gpu: torch.Tensor, kp_ref: torch.Tensor,
                   vp_ref: torch.Tensor) -> int:
    """Number of differing bytes over every slot except the dummy page's."""
    n = w.num_slots
    kb = kp_gpu[:n].cpu().contiguous().view(torch.uint8)
    vb = vp_gpu[:n].cpu().contiguous().view(torch.uint8)
    return int((kb != kp_ref[:n].contiguous().view(torch.uint8)).sum()) + \
        int((vb != vp_ref[:n].contiguous().view(torch.uint8)).sum())


def max_abs(out_gpu: torch.Tensor, ref: torch.Tensor) -> float:
    d = (out_gpu.detach().cpu().to(torch.float64) - ref).abs()
    if torch.isnan(d).any():
        return float("inf")
    return float(d.max()) if d.numel() else 0.0


def rowsum_error(w, kp_ref, vp_ref, lse_gpu: torch.Tensor, requests: Sequence[int]) -> float:
    """max |sum_j exp(s_j - lse) - 1| over the given requests' query rows and
    heads, with s_j recomputed in fp64 on the host from the post-store pool
    (q head h reads kv head h // (H / G))."""
    lse = lse_gpu.detach().cpu().to(torch.float64)
    H, G, d = w.q_heads, w.kv_heads, w.head_dim
    g = H // G
    worst = 0.0
    q = w.q.detach().cpu().to(torch.float64)
    seq_lens, cu_q, table_idx = w.seq_lens.cpu(), w.cu_q.cpu(), w.table_idx.cpu()
    page_table = w.page_table.cpu()
    for b in requests:
        L = int(seq_lens[b])
        c0, c1 = int(cu_q[b]), int(cu_q[b + 1])
        row = page_table[int(table_idx[b]), :L].long()
        K = kp_ref[row].to(torch.float64)  # [L, G, d]
        for t in range(c0, c1):
            p = L - (c1 - c0) + (t - c0)
            s = torch.einsum("jgd,gkd->gkj", K[:p + 1], q[t].view(G, g, d)) / math.sqrt(d)  # [G, g, p+1]
            tot = torch.exp(s - lse[t].view(G, g, 1)).sum(dim=2)
            worst = max(worst, float((tot - 1.0).abs().max()))
    return worst


def sample_rows(w, n: int, seed: int = 0) -> np.ndarray:
    """Query rows to check at full size: each request's first and last row plus
    random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.bs):
        rows.add(int(w.cu_q[b]))
        rows.add(int(w.cu_q[b + 1]) - 1)
    extra = rng.choice(w.num_tokens, size=min(n, w.num_tokens), replace=False)
    rows.update(int(x) for x in extra)
    return np.array(sorted(rows))


def oracle_rows(oracle, w, kp_ref, vp_ref, rows: np.ndarray):
    """Oracle output for selected query rows: each row becomes a one-query
    request at its own position (same page-table row, same keys)."""
    cu = w.cu_q.cpu().numpy()
    b_of = np.searchsorted(cu, rows, side="right") - 1
    L = w.seq_lens.cpu().numpy()
    C = w.cached_lens.cpu().numpy()
    pos = C[b_of] + (rows - cu[b_of])
    assert np.all(pos < L[b_of])
    tix = torch.from_numpy(w.table_idx.cpu().numpy()[b_of].astype(np.int32))
    seq = torch.from_numpy((pos + 1).astype(np.int32))
    qs = torch.arange(len(rows) + 1, dtype=torch.int32)
    q = w.q.cpu()[torch.from_numpy(rows)]
    return oracle.attention(q, kp_ref, vp_ref, w.page_table.cpu(), tix, seq, qs)
