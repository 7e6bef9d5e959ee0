"""Seeded synthetic inputs for the paged-KV attention step.

This module builds inputs only: lengths, free lists, page tables, the batch
metadata the engine derives from them (positions, out_loc, query offsets), and
K/V/Q values.  It holds none of the attention arithmetic; both the HIP path and
the oracle consume what it produces.

Conventions taken from the pages:

* Pool shape per layer is ``(num_pages + 1, page_size, kv_heads, head_dim)``:
  one page beyond the usable ones is reserved for the dummy request
  ("Engine and sampler", section on initialisation order; the stage-4 milestone
  prints ``(257, 1, 8, 128)`` for 256 pages).  Here it is flattened to
  ``[num_slots_total, kv_heads, head_dim]`` with slot = page * page_size + offset.
* ``page_table`` is int32 ``[max_running_req + 1, align_up_32(max_seq_len)]``;
  row r holds the KV slot of every token of the request in row r, and the last
  row belongs to the dummy request and is filled with the dummy page's first
  slot (same section; the hand-driven engine prints ``(5, 256)``).
* For a request with ``cached_len`` C and ``device_len`` L the step's new tokens
  sit at positions ``C .. L-1`` and are written to
  ``out_loc = page_table[row, C:L]`` (stage-4 milestone script and the
  hand-driven engine in "Engine and sampler").

Values are drawn by a counter-based generator: every element is
``table[h(seed, stream, index) >> 16]`` where ``table`` holds the 65536
mid-point quantiles of the target normal distribution (already rounded to the
storage dtype) and ``h`` is a 32-bit integer mixer.  The generator is pure
integer work, so it gives identical bits on the CPU and on the GPU, which lets
large pools be filled in device memory while any sampled slice can be rebuilt
on the host.  K/V values are indexed by the *logical* token (request, position),
then placed at their slot, so permuting slots or changing the page size leaves
the logical contents unchanged.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

# ----------------------------------------------------------------------------
# counter-based value generator
# ----------------------------------------------------------------------------

_M32 = 0xFFFFFFFF
_MUL1 = 0x7FEB352D
_MUL2 = 0x846CA68B

STREAM_K = 1
STREAM_V = 2
STREAM_Q = 3
STREAM_EMBED = 1 << 20  # vocabulary table values (a stream no layer's K/V/Q uses)


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding values < 2**32.

    The constant is split into 16-bit halves so that no intermediate product
    exceeds 2**48 (no signed overflow anywhere)."""
    lo = c & 0xFFFF
    hi = c >> 16
    return ((x * lo) + (((x * hi) & 0xFFFF) << 16)) & _M32


def _mix32_t(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, _MUL1)
    x = x ^ (x >> 15)
    x = _mul32(x, _MUL2)
    x = x ^ (x >> 16)
    return x


def _mix32_i(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * _MUL1) & _M32
    x ^= x >> 15
    x = (x * _MUL2) & _M32
    x ^= x >> 16
    return x


def stream_key(seed: int, stream: int) -> int:
    return _mix32_i(_mix32_i(seed * 0x9E3779B1 + 0x632BE5AB) ^ (stream * 0x85EBCA77))


def hash_u16(seed: int, stream: int, idx: torch.Tensor) -> torch.Tensor:
    """16-bit hash of int64 element indices (any device)."""
    key = stream_key(seed, stream)
    lo = idx & _M32
    hi = idx >> 32
    h = _mix32_t(lo ^ key)
    h = _mix32_t(h ^ _mul32(hi + 1, 0x27D4EB2F) ^ ((key * 0x165667B1) & _M32))
    return h >> 16


_TABLE_CACHE = {}


def normal_table(std: float, dtype: torch.dtype) -> torch.Tensor:
    """65536 mid-point quantiles of N(0, std**2), rounded once (RNE) to ``dtype``,
    returned as float32 holding exactly representable values."""
    key = (float(std), dtype)
    t = _TABLE_CACHE.get(key)
    if t is None:
        from scipy.special import ndtri

        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        vals = ndtri(u) * std
        t = torch.from_numpy(vals).to(torch.float32)
        if dtype == torch.bfloat16:
            t = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32)
        _TABLE_CACHE[key] = t
    return t


def gen_values(seed: int, stream: int, start: int, count: int, std: float,
               dtype: torch.dtype, device, chunk: int = 1 << 26) -> torch.Tensor:
    """Elements ``start .. start+count-1`` of one value stream, as ``dtype``."""
    table = normal_table(std, dtype).to(device)
    out = torch.empty(count, dtype=dtype, device=device)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        idx = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=device)
        out[c0:c0 + n] = table[hash_u16(seed, stream, idx)].to(dtype)
    return out


def gen_rows(seed: int, stream: int, rows: torch.Tensor, row_elems: int, std: float,
             dtype: torch.dtype, device, chunk_rows: int = 1 << 16) -> torch.Tensor:
    """Values for the given logical row ids (int64 tensor), ``[len(rows), row_elems]``."""
    table = normal_table(std, dtype).to(device)
    rows = rows.to(device=device, dtype=torch.int64)
    out = torch.empty(rows.numel(), row_elems, dtype=dtype, device=device)
    col = torch.arange(row_elems, dtype=torch.int64, device=device)
    for r0 in range(0, rows.numel(), chunk_rows):
        r = rows[r0:r0 + chunk_rows]
        idx = r[:, None] * row_elems + col[None, :]
        out[r0:r0 + r.numel()] = table[hash_u16(seed, stream, idx)].to(dtype)
    return out


# ----------------------------------------------------------------------------
# batch structure
# ----------------------------------------------------------------------------


def align_up_32(n: int) -> int:
    return (n + 31) // 32 * 32


def kv_bytes_per_token(head_dim: int, kv_heads: int, itemsize: int, num_layers: int) -> int:
    """K and V bytes one token occupies over all layers (the pages' per-page
    byte count at page_size 1: 2 x head_dim x kv_heads x itemsize x layers)."""
    return 2 * head_dim * kv_heads * itemsize * num_layers


def pool_shape(num_pages: int, page_size: int, kv_heads: int, head_dim: int):
    """Per-layer pool shape with the extra dummy page, as the engine allocates it."""
    return (num_pages + 1, page_size, kv_heads, head_dim)


def page_table_shape(max_running_req: int, max_seq_len: int):
    """Page-table shape with the extra dummy row."""
    return (max_running_req + 1, align_up_32(max_seq_len))


@dataclasses.dataclass
class Workload:
    name: str
    mode: str                  # "decode" or "prefill"
    dtype: torch.dtype         # storage dtype of q / pools / out
    q_heads: int
    kv_heads: int
    head_dim: int
    page_size: int
    num_slots: int             # usable slots (the dummy page follows)
    max_running_req: int
    max_seq_len: int
    page_table: torch.Tensor   # int32 [R+1, W]
    table_idx: torch.Tensor    # int32 [bs]
    seq_lens: torch.Tensor     # int32 [bs]   device_len (includes the new tokens)
    cached_lens: torch.Tensor  # int32 [bs]
    cu_q: torch.Tensor         # int32 [bs+1] offsets of each request's new tokens
    positions: torch.Tensor    # int32 [T]
    out_loc: torch.Tensor      # int32 [T]
    k_pool: torch.Tensor       # [S_total, G, d] state before store_kv
    v_pool: torch.Tensor
    k_new: torch.Tensor        # [T, G, d]
    v_new: torch.Tensor
    q: torch.Tensor            # [T, H, d]
    seed: int = 0
    layer: int = 0

    @property
    def bs(self) -> int:
        return int(self.table_idx.numel())

    @property
    def num_tokens(self) -> int:
        return int(self.out_loc.numel())

    @property
    def num_slots_total(self) -> int:
        return self.num_slots + self.page_size

    @property
    def dummy_slot(self) -> int:
        return self.num_slots

    @property
    def row_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def to(self, device) -> "Workload":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)

    def kv_bytes_read(self) -> int:
        """K+V bytes the attention step reads (each visible token once per kv head)."""
        e = torch.finfo(self.dtype).bits // 8
        return int(self.seq_lens.to(torch.int64).sum().item()) * self.kv_heads * self.head_dim * 2 * e


def _build_metadata(page_table: torch.Tensor, table_idx, seq_lens, cached_lens):
    """positions / out_loc / cu_q for the step, as the hand-driven engine builds them."""
    ext = [int(L) - int(C) for L, C in zip(seq_lens, cached_lens)]
    cu = np.zeros(len(ext) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(ext)
    pos = np.concatenate([np.arange(int(C), int(L)) for L, C in zip(seq_lens, cached_lens)]) \
        if ext else np.zeros(0, dtype=np.int64)
    pt = page_table.numpy()
    loc = np.concatenate([pt[int(r), int(C):int(L)] for r, L, C in zip(table_idx, seq_lens, cached_lens)]) \
        if ext else np.zeros(0, dtype=np.int64)
    return (torch.from_numpy(cu.astype(np.int32)), torch.from_numpy(pos.astype(np.int32)),
            torch.from_numpy(loc.astype(np.int32)))


def _fill(seed, layer, slots_hist, tok_hist, tok_new, t_q, G, H, d, dtype, kv_std, q_std,
          num_slots_total, device):
    """Pools with history placed at their slots; new K/V rows; Q."""
    rowe = G * d
    k_pool = torch.zeros(num_slots_total, G, d, dtype=dtype, device=device)
    v_pool = torch.zeros(num_slots_total, G, d, dtype=dtype, device=device)
    sk = STREAM_K + 4 * layer
    sv = STREAM_V + 4 * layer
    sq = STREAM_Q + 4 * layer
    if tok_hist.numel():
        sl = slots_hist.to(device=device, dtype=torch.int64)
        for r0 in range(0, tok_hist.numel(), 1 << 18):
            r = tok_hist[r0:r0 + (1 << 18)]
            k_pool.view(-1, rowe)[sl[r0:r0 + r.numel()]] = gen_rows(seed, sk, r, rowe, kv_std, dtype, device)
            v_pool.view(-1, rowe)[sl[r0:r0 + r.numel()]] = gen_rows(seed, sv, r, rowe, kv_std, dtype, device)
    k_new = gen_rows(seed, sk, tok_new, rowe, kv_std, dtype, device).view(-1, G, d)
    v_new = gen_rows(seed, sv, tok_new, rowe, kv_std, dtype, device).view(-1, G, d)
    q = gen_rows(seed, sq, torch.arange(t_q, dtype=torch.int64), H * d, q_std, dtype, device).view(-1, H, d)
    return k_pool, v_pool, k_new, v_new, q


def build_workload(name: str, mode: str, dtype: torch.dtype, H: int, G: int, d: int,
                   page_size: int, num_slots: int, max_running_req: int, max_seq_len: int,
                   rows: List[np.ndarray], seq_lens, cached_lens, seed: int,
                   kv_std: float = 1.0, q_std: float = 1.0, layer: int = 0,
                   device="cpu", table_idx=None) -> Workload:
    """Assemble a workload from per-request slot rows (token-level slot ids for
    positions 0..L-1) and lengths."""
    R = max_running_req
    W = align_up_32(max_seq_len)
    pt = torch.zeros(R + 1, W, dtype=torch.int32)
    bs = len(seq_lens)
    if table_idx is None:
        table_idx = list(range(bs))
    for b in range(bs):
        row = np.asarray(rows[b])
        pt[table_idx[b], :row.size] = torch.from_numpy(row.astype(np.int32))
    pt[R, :] = num_slots  # dummy row points at the dummy page's first slot
    seq = torch.tensor([int(x) for x in seq_lens], dtype=torch.int32)
    cac = torch.tensor([int(x) for x in cached_lens], dtype=torch.int32)
    tix = torch.tensor([int(x) for x in table_idx], dtype=torch.int32)
    cu_q, positions, out_loc = _build_metadata(pt, tix, seq, cac)
    # logical token ids: request b's position j is token tok_base[b] + j
    Ls = np.asarray([int(x) for x in seq_lens], dtype=np.int64)
    tok_base = np.zeros(bs + 1, dtype=np.int64)
    tok_base[1:] = np.cumsum(Ls)
    hist_tok, hist_slot, new_tok = [], [], []
    for b in range(bs):
        C = int(cached_lens[b])
        L = int(Ls[b])
        row = np.asarray(rows[b], dtype=np.int64)
        hist_tok.append(tok_base[b] + np.arange(C))
        hist_slot.append(row[:C])
        new_tok.append(tok_base[b] + np.arange(C, L))
    cat = lambda xs: torch.from_numpy(np.concatenate(xs) if xs else np.zeros(0, np.int64))
    k_pool, v_pool, k_new, v_new, q = _fill(
        seed, layer, cat(hist_slot), cat(hist_tok), cat(new_tok), int(out_loc.numel()),
        G, H, d, dtype, kv_std, q_std, num_slots + page_size, device)
    dev = lambda t: t.to(device)
    return Workload(name=name, mode=mode, dtype=dtype, q_heads=H, kv_heads=G, head_dim=d,
                    page_size=page_size, num_slots=num_slots, max_running_req=R,
                    max_seq_len=max_seq_len, page_table=dev(pt), table_idx=dev(tix),
                    seq_lens=dev(seq), cached_lens=dev(cac), cu_q=dev(cu_q),
                    positions=dev(positions), out_loc=dev(out_loc), k_pool=k_pool,
                    v_pool=v_pool, k_new=k_new, v_new=v_new, q=q, seed=seed, layer=layer)


# ----------------------------------------------------------------------------
# slot assignment
# ----------------------------------------------------------------------------


def rows_from_free_slots(free: np.ndarray, lens, cached=None, new_after_history=True):
    """Token-level slot rows at page_size 1 from a shuffled free list.

    Decode layout (``new_after_history``): every request pops its history
    slots first, in request order, and the step's new tokens then take the
    next free slots, one block per request, so the new tokens land on random
    free slots just as a scheduler would hand them out."""
    rows = []
    pos = 0
    lens = [int(x) for x in lens]
    if cached is None:
        cached = [L - 1 for L in lens]
    if new_after_history:
        hist = []
        for L, C in zip(lens, cached):
            hist.append(free[pos:pos + C])
            pos += C
        for (L, C), h in zip(zip(lens, cached), hist):
            rows.append(np.concatenate([h, free[pos:pos + (L - C)]]))
            pos += L - C
    else:
        for L in lens:
            rows.append(free[pos:pos + L])
            pos += L
    assert pos <= free.size, "pool too small for the batch"
    return rows


def rows_from_free_pages(free_pages: np.ndarray, lens, page_size: int):
    """Token-level slot rows at page_size > 1: request b takes ceil(L/ps) pages
    from the shuffled free-page list; token j sits at page[j // ps] * ps + j % ps."""
    rows = []
    pos = 0
    for L in lens:
        L = int(L)
        n = (L + page_size - 1) // page_size
        pages = free_pages[pos:pos + n].astype(np.int64)
        pos += n
        j = np.arange(L)
        rows.append(pages[j // page_size] * page_size + j % page_size)
    assert pos <= free_pages.size, "pool too small for the batch"
    return rows


def lognormal_lengths(rng: np.random.Generator, n: int, median: float = 2048.0,
                      sigma: float = 1.0, lo: int = 16, hi: int = 32768) -> np.ndarray:
    x = np.round(np.exp(rng.normal(math.log(median), sigma, size=n)))
    return np.clip(x, lo, hi).astype(np.int64)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

QWEN3_06B = dict(H=16, G=8, d=128)
QWEN3_8B = dict(H=32, G=8, d=128)


def tiny(mode: str = "decode", seed: int = 1001, device="cpu", lens=(5, 9),
         H: int = 4, G: int = 2, d: int = 64, num_slots: int = 256,
         dtype: torch.dtype = torch.float32) -> Workload:
    """Tiny single layer: fp32, page_size 1, 2 requests of 5 and 9 tokens,
    4 q heads / 2 kv heads / head_dim 64, a 256-slot pool.  Each page-table row
    is a full random permutation of the slot ids, with live prefixes disjoint
    across rows.  Q/K/V ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    rows = []
    used = np.zeros(num_slots, dtype=bool)
    for L in lens:
        free = np.flatnonzero(~used)
        taken = np.flatnonzero(used)
        row = np.concatenate([rng.permutation(free), rng.permutation(taken)])
        used[row[:L]] = True
        rows.append(row)
    cached = [L - 1 for L in lens] if mode == "decode" else [0] * len(lens)
    return build_workload(f"tiny-{mode}", mode, dtype, H, G, d, 1, num_slots, len(lens),
                          num_slots, rows, lens, cached, seed, 1.0, 1.0, device=device)


def qwen3_06b_decode(seed: int = 1002, device="cpu", bs: int = 64, lo: int = 512, hi: int = 4096,
                     num_slots: int = 1 << 19, q_std: Optional[float] = None,
                     dtype: torch.dtype = torch.bfloat16) -> Workload:
    """Qwen3-0.6B-shaped decode (16q/8kv, d128, bf16), page_size 1, batch 64,
    context lengths U[512, 4096]; slots from a shuffled free list; the batch's
    new tokens take random free slots."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=bs, endpoint=True)
    free = rng.permutation(num_slots)
    rows = rows_from_free_slots(free, lens)
    cached = [int(L) - 1 for L in lens]
    return build_workload("qwen3-0.6b-decode", "decode", dtype, **QWEN3_06B, page_size=1,
                          num_slots=num_slots, max_running_req=bs, max_seq_len=hi, rows=rows,
                          seq_lens=lens, cached_lens=cached, seed=seed, kv_std=1.0,
                          q_std=q_std if q_std is not None else 1.0 / math.sqrt(128), device=device)


def ragged_prefill(seed: int = 1003, device="cpu", n_req: int = 8, e_lo: int = 128, e_hi: int = 2048,
                   c_lo: int = 0, c_hi: int = 1024, num_slots: int = 1 << 15,
                   q_std: Optional[float] = None, dtype: torch.dtype = torch.bfloat16,
                   heads=QWEN3_06B, page_size: int = 1) -> Workload:
    """Ragged causal prefill/extend (16q/8kv, d128, bf16): 8 requests, extend
    lengths U[128, 2048] on a resident cached prefix U[0, 1024]; shuffled free
    list, each request's prefix slots first, then its new tokens (at page size
    > 1: shuffled free pages, each request's tokens in page order)."""
    rng = np.random.default_rng(seed)
    ext = rng.integers(e_lo, e_hi, size=n_req, endpoint=True)
    cac = rng.integers(c_lo, c_hi, size=n_req, endpoint=True)
    lens = ext + cac
    if page_size == 1:
        free = rng.permutation(num_slots)
        rows = rows_from_free_slots(free, lens, new_after_history=False)
    else:
        rows = rows_from_free_pages(rng.permutation(num_slots // page_size), lens, page_size)
    return build_workload("ragged-prefill", "prefill", dtype, **heads, page_size=page_size,
                          num_slots=num_slots, max_running_req=n_req, max_seq_len=c_hi + e_hi,
                          rows=rows, seq_lens=lens, cached_lens=cac, seed=seed, kv_std=1.0,
                          q_std=q_std if q_std is not None else 1.0 / math.sqrt(128), device=device)


def qwen3_8b_decode(page_size: int = 1, seed: int = 1004, device="cpu", bs: int = 256,
                    num_slots: int = 1 << 21, median: float = 2048.0, hi: int = 32768,
                    q_std: Optional[float] = None, dtype: torch.dtype = torch.bfloat16,
                    heads=QWEN3_8B, max_running_req: Optional[int] = None) -> Workload:
    """Qwen3-8B-shaped decode (32q/8kv, d128, bf16), batch 256, lognormal
    context lengths (median 2048, sigma 1) clipped to [16, 32768], at
    page_size 1 (shuffled free slots) or 16 (shuffled free pages).  Lengths are
    drawn first, so both page sizes see the same logical K/V."""
    rng = np.random.default_rng(seed)
    lens = lognormal_lengths(rng, bs, median=median, hi=hi)
    if page_size == 1:
        free = rng.permutation(num_slots)
        rows = rows_from_free_slots(free, lens)
    else:
        free_pages = rng.permutation(num_slots // page_size)
        rows = rows_from_free_pages(free_pages, lens, page_size)
    cached = [int(L) - 1 for L in lens]
    return build_workload(f"qwen3-8b-decode-ps{page_size}", "decode", dtype, **heads,
                          page_size=page_size, num_slots=num_slots,
                          max_running_req=max_running_req or bs, max_seq_len=hi,
                          rows=rows, seq_lens=lens, cached_lens=cached, seed=seed, kv_std=1.0,
                          q_std=q_std if q_std is not None else 1.0 / math.sqrt(128), device=device)


# ----------------------------------------------------------------------------
# graph padding
# ----------------------------------------------------------------------------

GRAPH_BATCH_SIZES = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def padded_batch_size(bs: int, sizes=GRAPH_BATCH_SIZES) -> int:
    """Smallest recorded batch size that holds ``bs`` (3 -> 4 in the pages' replay)."""
    for s in sizes:
        if s >= bs:
            return s
    raise ValueError(f"batch {bs} exceeds the largest recorded size {sizes[-1]}")


def subset_decode(w: Workload, n: int) -> Workload:
    """The first ``n`` requests of a decode workload (same pools and table)."""
    assert w.mode == "decode"
    return dataclasses.replace(
        w, table_idx=w.table_idx[:n].clone(), seq_lens=w.seq_lens[:n].clone(),
        cached_lens=w.cached_lens[:n].clone(), cu_q=w.cu_q[:n + 1].clone(),
        positions=w.positions[:n].clone(), out_loc=w.out_loc[:n].clone(),
        k_new=w.k_new[:n].clone(), v_new=w.v_new[:n].clone(), q=w.q[:n].clone())


def pad_decode(w: Workload, padded_bs: int) -> Workload:
    """Pad a decode batch with dummy requests: each uses the dummy page-table
    row, has one token (seq_len 1, cached 0) and writes the dummy slot; its
    outputs are discarded."""
    assert w.mode == "decode"
    bs = w.bs
    extra = padded_bs - bs
    assert extra >= 0
    if extra == 0:
        return w
    dev = w.q.device
    i32 = lambda v: torch.full((extra,), v, dtype=torch.int32, device=dev)
    cat = lambda a, b: torch.cat([a, b])
    return dataclasses.replace(
        w,
        table_idx=cat(w.table_idx, i32(w.max_running_req)),
        seq_lens=cat(w.seq_lens, i32(1)),
        cached_lens=cat(w.cached_lens, i32(0)),
        cu_q=torch.arange(padded_bs + 1, dtype=torch.int32, device=dev),
        positions=cat(w.positions, i32(0)),
        out_loc=cat(w.out_loc, i32(w.dummy_slot)),
        k_new=cat(w.k_new, torch.zeros(extra, w.kv_heads, w.head_dim, dtype=w.dtype, device=dev)),
        v_new=cat(w.v_new, torch.zeros(extra, w.kv_heads, w.head_dim, dtype=w.dtype, device=dev)),
        q=cat(w.q, torch.zeros(extra, w.q_heads, w.head_dim, dtype=w.dtype, device=dev)),
    )


# ----------------------------------------------------------------------------
# the mixed multi-layer step
# ----------------------------------------------------------------------------

MIXED_POOL_FRACTION = 0.6
MIXED_HBM_BYTES = 288e9


@dataclasses.dataclass
class MixedStep:
    """One engine step over `layers` layers: decode requests plus chunked
    prefills in one batch.  All layers share the page table and metadata (one
    free list, the same slots in every layer); each layer has its own pools,
    new K/V rows and queries.  `decode` and `prefill` are per-layer workload
    views (layer 0 here); `layer_inputs(l)` returns layer l's tensors."""
    decode: Workload
    prefill: Workload
    layers: int
    k_pools: List[torch.Tensor]
    v_pools: List[torch.Tensor]
    k_new: List[torch.Tensor]      # [T_decode + T_prefill, G, d] per layer
    v_new: List[torch.Tensor]
    q: List[torch.Tensor]          # [T_decode + T_prefill, H, d] per layer
    out_loc: torch.Tensor          # [T_decode + T_prefill]

    @property
    def num_tokens(self) -> int:
        return int(self.out_loc.numel())

    def layer_views(self, layer: int):
        """(decode, prefill) workload views bound to one layer's tensors."""
        nd = self.decode.num_tokens
        d = dataclasses.replace(self.decode, k_pool=self.k_pools[layer], v_pool=self.v_pools[layer],
                                k_new=self.k_new[layer][:nd], v_new=self.v_new[layer][:nd],
                                q=self.q[layer][:nd], layer=layer)
        p = dataclasses.replace(self.prefill, k_pool=self.k_pools[layer], v_pool=self.v_pools[layer],
                                k_new=self.k_new[layer][nd:], v_new=self.v_new[layer][nd:],
                                q=self.q[layer][nd:], layer=layer)
        return d, p


def mixed_step(seed: int = 1005, device="cpu", layers: int = 36, n_decode: int = 192,
               n_chunks: int = 2, chunk: int = 2048, prefix: int = 8192,
               num_slots: Optional[int] = None, median: float = 2048.0, hi: int = 32768,
               heads=QWEN3_8B, dtype: torch.dtype = torch.bfloat16) -> MixedStep:
    """The mixed step: `n_decode` decode requests (lognormal contexts as in the
    Qwen3-8B decode workload) and `n_chunks` chunked prefills of `chunk` new
    tokens on a `prefix`-token cached prefix, over `layers` layers of Qwen3-8B
    attention shapes.  The pool holds 60% of 288 GB (decimal) across all layers
    at page_size 1: 0.6 * 288e9 / (layers * 2 * kv_heads * head_dim * 2 bytes)
    slots per layer; one shuffled free list serves every layer."""
    H, G, d = heads["H"], heads["G"], heads["d"]
    e = torch.finfo(dtype).bits // 8
    if num_slots is None:
        num_slots = int(MIXED_POOL_FRACTION * MIXED_HBM_BYTES) // (layers * 2 * G * d * e)
    rng = np.random.default_rng(seed)
    dec_lens = lognormal_lengths(rng, n_decode, median=median, hi=hi)
    free = rng.permutation(num_slots)
    # decode requests: history then their new token; chunks: prefix then new tokens
    dec_rows = rows_from_free_slots(free, dec_lens)
    used = int(dec_lens.sum())
    pre_lens = np.full(n_chunks, prefix + chunk, dtype=np.int64)
    pre_rows = rows_from_free_slots(free[used:], pre_lens, new_after_history=False)
    R = n_decode + n_chunks
    W = align_up_32(max(hi, prefix + chunk))
    pt = torch.zeros(R + 1, W, dtype=torch.int32)
    for b, row in enumerate(dec_rows + pre_rows):
        pt[b, :row.size] = torch.from_numpy(np.asarray(row).astype(np.int32))
    pt[R, :] = num_slots
    dec_cached = [int(L) - 1 for L in dec_lens]
    pre_cached = [prefix] * n_chunks
    lens = [int(x) for x in dec_lens] + [int(x) for x in pre_lens]
    cached = dec_cached + pre_cached
    tix = list(range(R))
    # logical tokens of the whole step (decode requests first)
    Ls = np.asarray(lens, dtype=np.int64)
    tok_base = np.zeros(R + 1, dtype=np.int64)
    tok_base[1:] = np.cumsum(Ls)
    rows_all = dec_rows + pre_rows
    hist_tok = torch.from_numpy(np.concatenate([tok_base[b] + np.arange(cached[b]) for b in range(R)]))
    hist_slot = torch.from_numpy(np.concatenate([np.asarray(rows_all[b][:cached[b]], dtype=np.int64)
                                                 for b in range(R)]))
    new_tok = torch.from_numpy(np.concatenate([tok_base[b] + np.arange(cached[b], lens[b]) for b in range(R)]))

    def meta(sel):
        t_idx = torch.tensor([tix[b] for b in sel], dtype=torch.int32)
        s = torch.tensor([lens[b] for b in sel], dtype=torch.int32)
        c = torch.tensor([cached[b] for b in sel], dtype=torch.int32)
        cu, pos, loc = _build_metadata(pt, t_idx, s, c)
        return t_idx, s, c, cu, pos, loc

    k_pools, v_pools, k_news, v_news, qs = [], [], [], [], []
    for layer in range(layers):
        kp, vp, kn, vn, q = _fill(seed, layer, hist_slot, hist_tok, new_tok, int(new_tok.numel()), G, H, d,
                                  dtype, 1.0, 1.0 / math.sqrt(128), num_slots + 1, device)
        k_pools.append(kp)
        v_pools.append(vp)
        k_news.append(kn)
        v_news.append(vn)
        qs.append(q)
    views = []
    nd_tokens = n_decode
    for sel, mode, sl in ((range(n_decode), "decode", slice(0, nd_tokens)),
                          (range(n_decode, R), "prefill", slice(nd_tokens, None))):
        t_idx, s, c, cu, pos, loc = meta(list(sel))
        views.append(Workload(
            name=f"mixed-{mode}", mode=mode, dtype=dtype, q_heads=H, kv_heads=G, head_dim=d, page_size=1,
            num_slots=num_slots, max_running_req=R, max_seq_len=W, page_table=pt.to(device),
            table_idx=t_idx.to(device), seq_lens=s.to(device), cached_lens=c.to(device), cu_q=cu.to(device),
            positions=pos.to(device), out_loc=loc.to(device), k_pool=k_pools[0], v_pool=v_pools[0],
            k_new=k_news[0][sl], v_new=v_news[0][sl], q=qs[0][sl], seed=seed, layer=0))
    out_loc = torch.cat([views[0].out_loc, views[1].out_loc])
    return MixedStep(decode=views[0], prefill=views[1], layers=layers, k_pools=k_pools, v_pools=v_pools,
                     k_new=k_news, v_new=v_news, q=qs, out_loc=out_loc)


def layer_history_values(step: MixedStep, layer: int, request: int, positions: torch.Tensor, which: str):
    """Regenerate the K ('k') or V ('v') rows of one request's history positions
    in one layer, as the generator placed them (for spot checks of pools)."""
    w = step.decode if request < step.decode.bs else step.prefill
    lens = torch.cat([step.decode.seq_lens.cpu(), step.prefill.seq_lens.cpu()]).long()
    base = int(lens[:request].sum())
    stream = (STREAM_K if which == "k" else STREAM_V) + 4 * layer
    rows = base + positions.long().cpu()
    return gen_rows(w.seed, stream, rows, w.kv_heads * w.head_dim, 1.0, w.dtype, "cpu").view(
        -1, w.kv_heads, w.head_dim)


# ----------------------------------------------------------------------------
# vocabulary indexing
# ----------------------------------------------------------------------------

QWEN3_VOCAB = 151936
QWEN3_8B_HIDDEN = 4096


@dataclasses.dataclass
class VocabBatch:
    name: str
    weight: torch.Tensor   # [rows, hidden]: the vocabulary ids vocab_start .. vocab_start + rows - 1
    vocab_start: int
    vocab_size: int        # of the whole (unsharded) vocabulary
    ids: torch.Tensor      # int32 [T]

    @property
    def num_tokens(self) -> int:
        return int(self.ids.numel())

    @property
    def hidden(self) -> int:
        return int(self.weight.shape[1])


def vocab_batch(seed: int = 1006, device="cpu", num_tokens: int = 4288, vocab: int = QWEN3_VOCAB,
                hidden: int = QWEN3_8B_HIDDEN, shards: int = 1, rank: int = 0,
                dtype: torch.dtype = torch.bfloat16, std: float = 0.02) -> VocabBatch:
    """Token ids of one step (uniform over the whole vocabulary) and one rank's
    shard of an embedding table: rows [vocab * rank // shards, vocab * (rank+1)
    // shards) of a table whose row r holds stream values r * hidden .. (r+1) *
    hidden - 1 (N(0, std^2) quantiles).  Defaults: the Qwen3-8B table (151936 x
    4096, bf16) and the 4288 new tokens of the mixed step."""
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(rng.integers(0, vocab, size=num_tokens).astype(np.int32)).to(device)
    lo, hi = vocab * rank // shards, vocab * (rank + 1) // shards
    weight = gen_rows(seed, STREAM_EMBED, torch.arange(lo, hi, dtype=torch.int64), hidden, std, dtype, device)
    return VocabBatch(f"vocab-{vocab}x{hidden}-tp{shards}r{rank}", weight, lo, vocab, ids)


# ----------------------------------------------------------------------------
# decode over shared radix prefixes
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class SharedPrefixBatch:
    w: Workload                # the decode batch (every request's full page-table row)
    group_start: torch.Tensor  # int32 [groups + 1] batch rows of each group
    prefix_lens: torch.Tensor  # int32 [bs] shared prefix length of each request's group (0: none)
    max_group_size: int
    max_prefix_len: int


def shared_prefix_decode(seed: int = 1007, device="cpu", group_sizes=(64, 64, 64, 64),
                         prefixes=(4096, 4096, 4096, 4096), singles: int = 0, suffix_lo: int = 16,
                         suffix_hi: int = 1024, page_size: int = 1, num_slots: int = 1 << 20,
                         heads=QWEN3_8B, q_std: Optional[float] = None,
                         dtype: torch.dtype = torch.bfloat16) -> SharedPrefixBatch:
    """Decode batch whose requests come in groups that share a radix prefix:
    group g's requests hold the same slots for positions 0 .. prefixes[g]-1
    (taken once from the shuffled free list, or as whole free pages at
    page_size > 1, when the prefixes are page multiples), then their own
    suffix of U[suffix_lo, suffix_hi] tokens, the last of which is the step's
    new token.  `singles` more requests share nothing (prefix 0).  Defaults:
    Qwen3-8B heads, bf16, batch 256 in 4 groups of 64 on 4096-token prefixes.
    A shared slot's K/V values are those its group's last request writes."""
    assert len(group_sizes) == len(prefixes)
    rng = np.random.default_rng(seed)
    n_grouped = int(sum(group_sizes))
    bs = n_grouped + singles
    suffix = rng.integers(suffix_lo, suffix_hi, size=bs, endpoint=True)
    plen = np.zeros(bs, dtype=np.int64)
    gstart = [0]
    for n, P in zip(group_sizes, prefixes):
        plen[gstart[-1]:gstart[-1] + n] = P
        gstart.append(gstart[-1] + n)
    lens = plen + suffix
    rows = []
    if page_size == 1:
        free = rng.permutation(num_slots)
        pos = 0
        for g, (n, P) in enumerate(zip(group_sizes, prefixes)):
            shared = free[pos:pos + P]
            pos += P
            for b in range(gstart[g], gstart[g] + n):
                rows.append(np.concatenate([shared, free[pos:pos + suffix[b]]]))
                pos += int(suffix[b])
        for b in range(n_grouped, bs):
            rows.append(free[pos:pos + suffix[b]])
            pos += int(suffix[b])
        assert pos <= num_slots, "pool too small for the batch"
    else:
        assert all(P % page_size == 0 for P in prefixes), "shared prefixes are whole pages"
        free_pages = rng.permutation(num_slots // page_size)
        pos = 0

        def take(n_tok):
            nonlocal pos
            n = (n_tok + page_size - 1) // page_size
            pages = free_pages[pos:pos + n].astype(np.int64)
            pos += n
            j = np.arange(n_tok)
            return pages[j // page_size] * page_size + j % page_size

        for g, (n, P) in enumerate(zip(group_sizes, prefixes)):
            shared = take(P)
            for b in range(gstart[g], gstart[g] + n):
                rows.append(np.concatenate([shared, take(int(suffix[b]))]))
        for b in range(n_grouped, bs):
            rows.append(take(int(suffix[b])))
        assert pos <= free_pages.size, "pool too small for the batch"
    cached = [int(L) - 1 for L in lens]
    max_len = int(lens.max())
    w = build_workload(f"shared-prefix-decode-ps{page_size}", "decode", dtype, **heads, page_size=page_size,
                       num_slots=num_slots, max_running_req=bs, max_seq_len=align_up_32(max_len + 1),
                       rows=rows, seq_lens=lens, cached_lens=cached, seed=seed, kv_std=1.0,
                       q_std=q_std if q_std is not None else 1.0 / math.sqrt(128), device=device)
    return SharedPrefixBatch(w, torch.tensor(gstart, dtype=torch.int32, device=device),
                             torch.from_numpy(plen.astype(np.int32)).to(device),
                             max(group_sizes) if group_sizes else 1, max(prefixes) if prefixes else 0)
