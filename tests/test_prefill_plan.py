"""Host plan of the prefill launch (msgl_prefill_plan): pure host code, run
here without a GPU.  The block list is checked against its definition
recomputed in Python: every (request, query block) pair exactly once, its key
tiles = ceil((cached + min((qb + 1) BQ, new)) / 64), the most tiles first and
ties in request order then query-block order, and the layout rule (the
single-block layout when requests average 2048 or more new tokens)."""

import ctypes
import math

import numpy as np
import pytest
import torch

FAKE = 0x10000  # never dereferenced: the calls below are rejected or launch nothing


@pytest.fixture(scope="module")
def L():
    from paged_kv_attention_slots_amd import _lib

    return _lib


def _meta(ext, cac, rows=None, row_stride=None):
    ext = np.asarray(ext, dtype=np.int64)
    cac = np.asarray(cac, dtype=np.int64)
    n = len(ext)
    cu = np.concatenate([[0], np.cumsum(ext)]).astype(np.int32)
    seq = (ext + cac).astype(np.int32)
    ti = np.arange(n, dtype=np.int32)[::-1].copy()
    rows = n if rows is None else rows
    row_stride = int(seq.max()) if row_stride is None else row_stride
    return (torch.from_numpy(seq), torch.from_numpy(cac.astype(np.int32)), torch.from_numpy(cu),
            torch.from_numpy(ti), rows, row_stride)


def _expected(ext, cac, bq):
    items = []
    for b, (e, c) in enumerate(zip(ext, cac)):
        for qb in range(math.ceil(e / bq)):
            tiles = math.ceil((c + min((qb + 1) * bq, e)) / 64)
            items.append((-tiles, b, qb))
    return [(b, qb, -t) for t, b, qb in sorted(items)]


@pytest.mark.parametrize("H,G", [(16, 8), (32, 8), (8, 8), (64, 8)])
def test_plan_matches_definition(L, H, G):
    rng = np.random.default_rng(7 + H)
    ext = rng.integers(1, 700, size=23)
    cac = rng.integers(0, 900, size=23)
    seq, cl, cu, ti, rows, rs = _meta(ext, cac)
    plan = L.msgl_prefill_plan(seq, cl, cu, ti, rows, rs, H, G).numpy()
    g = H // G
    bq = 128 // g
    head = plan[:8]
    exp = _expected(ext, cac, bq)
    assert head[0] == 0x4D504C31 and head[1] == 0 and head[2] == bq
    assert list(head[3:8]) == [len(exp), 23, int(ext.sum()), H, G]
    ent = plan[8:].reshape(-1, 8)
    assert [(int(r[0]), int(r[1]), int(r[6])) for r in ent] == exp
    for r in ent:
        b = int(r[0])
        assert r[2] == ext[b] and r[3] == cac[b] and r[4] == cu[b] and r[5] == ti[b] and r[7] == 0
    assert plan.nbytes <= L.msgl_prefill_plan_bytes(23, int(ext.sum()), H, G)


def test_plan_config3_workload(L):
    from paged_kv_attention_slots_amd import runner, workloads as wl

    w = wl.ragged_prefill()  # 8 requests, extends U[128, 2048] on cached prefixes U[0, 1024]
    plan, _ = runner.prefill_plan(w)
    ext = (w.seq_lens - w.cached_lens).tolist()
    exp = _expected(ext, w.cached_lens.tolist(), 64)
    ent = plan[8:].view(-1, 8)
    assert [(int(r[0]), int(r[1]), int(r[6])) for r in ent] == exp
    assert int(plan[1]) == 0 and int(plan[2]) == 64


def test_plan_long_layout(L):
    # two requests of 2048 new tokens: the single-block layout, 256 / g tokens per block
    seq, cl, cu, ti, rows, rs = _meta([2048, 2048], [8192, 8192])
    plan = L.msgl_prefill_plan(seq, cl, cu, ti, rows, rs, 32, 8).numpy()
    assert plan[1] == 1 and plan[2] == 64 and plan[3] == 64
    assert [tuple(int(x) for x in r[[0, 1, 6]]) for r in plan[8:].reshape(-1, 8)] == \
        _expected([2048, 2048], [8192, 8192], 64)
    # just below the average: the two-blocks-per-CU layout
    seq, cl, cu, ti, rows, rs = _meta([2048, 2047], [0, 0])
    plan = L.msgl_prefill_plan(seq, cl, cu, ti, rows, rs, 32, 8).numpy()
    assert plan[1] == 0 and plan[2] == 32


def test_plan_many_requests_and_bound(L):
    # beyond the 1024 requests of the device enumeration; the size query bounds every batch
    rng = np.random.default_rng(3)
    for n, hi in [(1500, 6), (40, 1), (7, 129)]:
        ext = rng.integers(1, hi, size=n, endpoint=True)
        cac = rng.integers(0, 50, size=n)
        seq, cl, cu, ti, rows, rs = _meta(ext, cac)
        plan = L.msgl_prefill_plan(seq, cl, cu, ti, rows, rs, 16, 8)
        assert int(plan[3]) == sum(math.ceil(e / 64) for e in ext)
        assert plan.numel() * 4 <= L.msgl_prefill_plan_bytes(n, int(ext.sum()), 16, 8)


def test_plan_rejects_malformed(L):
    seq, cl, cu, ti, rows, rs = _meta([5, 9], [3, 0])
    ok = dict(rows=rows, row_stride=rs, q_heads=16, kv_heads=8)

    def plan(**kw):
        a = dict(seq_lens=seq, cached_lens=cl, cu_q=cu, table_idx=ti, **ok)
        a.update(kw)
        return L.msgl_prefill_plan(a["seq_lens"], a["cached_lens"], a["cu_q"], a["table_idx"], a["rows"],
                                   a["row_stride"], a["q_heads"], a["kv_heads"], a.get("head_dim", 128),
                                   a.get("dtype", L.MSGL_BF16))

    assert int(plan()[3]) == 2
    cases = [
        (dict(seq_lens=torch.tensor([8, 10], dtype=torch.int32)), L.MSGL_INVALID_ARG, "cached + step"),
        (dict(cu_q=torch.tensor([1, 5, 14], dtype=torch.int32)), L.MSGL_INVALID_ARG, "cu_q[0]"),
        (dict(cached_lens=torch.tensor([-1, 0], dtype=torch.int32)), L.MSGL_INVALID_ARG, "request 0"),
        (dict(row_stride=8), L.MSGL_INVALID_ARG, "row_stride"),
        (dict(table_idx=torch.tensor([0, 2], dtype=torch.int32)), L.MSGL_INVALID_ARG, "table row"),
        (dict(dtype=L.MSGL_F32), L.MSGL_UNSUPPORTED, "bf16"),
        (dict(head_dim=64), L.MSGL_UNSUPPORTED, "bf16"),
        (dict(q_heads=12, kv_heads=4), L.MSGL_UNSUPPORTED, "group size"),
    ]
    for kw, status, text in cases:
        with pytest.raises(L.MsglError) as e:
            plan(**kw)
        assert e.value.status == status and text in str(e.value), (kw, str(e.value))
    # a buffer one entry short
    buf = torch.zeros(8 + 8, dtype=torch.int32)
    st = L.lib.msgl_prefill_plan(buf.data_ptr(), buf.numel() * 4, seq.data_ptr(), cl.data_ptr(), cu.data_ptr(),
                                 ti.data_ptr(), 2, 14, rows, rs, 16, 8, 128, L.MSGL_BF16)
    assert st == L.MSGL_WORKSPACE_TOO_SMALL
    assert L.msgl_prefill_plan_bytes(2, 14, 12, 8) == 0 and L.msgl_prefill_plan_bytes(-1, 0, 16, 8) == 0


def test_planned_call_checks(L):
    seq, cl, cu, ti, rows, rs = _meta([5, 9], [3, 0])
    plan = L.msgl_prefill_plan(seq, cl, cu, ti, rows, rs, 16, 8)

    def run(p, H=16, G=8, nbytes=None, dtype=L.MSGL_BF16):
        return L.lib.msgl_prefill_attn_planned(FAKE, None, FAKE, FAKE, FAKE, 100, FAKE, rs, H, G, 128, 1, 0.1,
                                               dtype, p.data_ptr(), FAKE, p.numel() * 4 if nbytes is None else nbytes,
                                               None)

    bad = plan.clone()
    bad[0] = 0
    assert run(bad) == L.MSGL_INVALID_ARG and "header" in L.msgl_last_error()
    assert run(plan, H=32) == L.MSGL_INVALID_ARG and "other heads" in L.msgl_last_error()
    assert run(plan, nbytes=plan.numel() * 4 - 4) == L.MSGL_INVALID_ARG
    assert run(plan, dtype=L.MSGL_F32) == L.MSGL_UNSUPPORTED
    bad = plan.clone()
    bad[2] = 32  # tokens per block of another layout
    assert run(bad) == L.MSGL_INVALID_ARG
    # an empty batch: a plan of no entries launches nothing
    empty = L.msgl_prefill_plan(torch.zeros(0, dtype=torch.int32), torch.zeros(0, dtype=torch.int32),
                                torch.zeros(1, dtype=torch.int32), torch.zeros(0, dtype=torch.int32), 1, 16, 16, 8)
    assert int(empty[3]) == 0 and run(empty) == L.MSGL_OK
