"""Device-side metadata check (msgl_check_batch) against the host validator.

Valid batches of the benchmark shapes (ragged prefill, Qwen3-8B decode at page
sizes 1 and 16, padded decode with the dummy slot) raise nothing.  Each planted
violation sets its code, names the first failing request (and new token), and
is refused by msgl_validate_batch on host copies too.  Seeded random
corruptions (huge, negative and off-by-one values in every metadata array)
agree with the host validator on whether the batch is valid; every kernel read
stays in bounds whatever the values (the check's own contract).
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

INT_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module")
def mods():
    from paged_kv_attention_slots_amd import _lib, workloads as wl

    return _lib, wl


def _meta(w, out_loc=True):
    return dict(page_table=w.page_table.cpu(), table_idx=w.table_idx.cpu(), seq_lens=w.seq_lens.cpu(),
                cached_lens=w.cached_lens.cpu(), cu_q=w.cu_q.cpu(),
                out_loc=w.out_loc.cpu() if out_loc else None, max_seq_len=w.max_seq_len,
                num_slots=w.num_slots_total, page_size=w.page_size, dummy_slot=w.dummy_slot)


def _run(L, m):
    """Device result [codes, flagged requests, first request, first token] and the host verdict."""
    g = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in m.items()}
    seen = torch.full(((m["num_slots"] + 31) // 32,), -1, dtype=torch.int32, device="cuda")  # the call clears it
    res = L.msgl_check_batch(g["page_table"], g["table_idx"], g["seq_lens"], g["cached_lens"], g["cu_q"],
                             m["max_seq_len"], m["num_slots"], m["page_size"], out_loc=g["out_loc"],
                             dummy_slot=m["dummy_slot"], seen=seen)
    torch.cuda.synchronize()
    r = [int(x) for x in res.cpu()]
    try:
        L.msgl_validate_batch(m["page_table"], m["table_idx"], m["seq_lens"], m["cached_lens"], m["cu_q"],
                              m["max_seq_len"], m["num_slots"], m["page_size"], out_loc=m["out_loc"],
                              dummy_slot=m["dummy_slot"])
        host_ok = True
    except L.MsglError:
        host_ok = False
    return r, host_ok


def test_valid_benchmark_batches(mods):
    L, wl = mods
    cases = [("ragged prefill, 8 requests", wl.ragged_prefill(device="cuda")),
             ("Qwen3-8B decode bs 256 ps1", wl.qwen3_8b_decode(page_size=1, device="cuda")),
             ("Qwen3-8B decode bs 256 ps16", wl.qwen3_8b_decode(page_size=16, device="cuda"))]
    for name, w in cases:
        r, host_ok = _run(L, _meta(w))
        say(f"[check] {name}: {r}")
        assert host_ok and r == [0, 0, INT_MAX, INT_MAX], (name, r)
        del w
    # a padded decode batch repeats the dummy slot: allowed when named, a repeat when not
    w = wl.qwen3_8b_decode(page_size=16, bs=5, num_slots=1 << 12, median=100.0, hi=512, device="cuda")
    p = wl.pad_decode(w, 8)
    m = _meta(p)
    m["dummy_slot"] = w.dummy_slot
    r, host_ok = _run(L, m)
    assert host_ok and r == [0, 0, INT_MAX, INT_MAX], r
    m["dummy_slot"] = -1
    r, host_ok = _run(L, m)
    # the three padding rows share the dummy slot: whichever two of them record it second and third are
    # flagged (atomic order), so the first flagged request is 5 or 6
    assert not host_ok and r[0] == L.CHECK_CODES["repeat"] and r[1] == 2 and r[2] in (5, 6), r


def _token_owner(m, t):
    cu = m["cu_q"].tolist()
    return max(b for b in range(len(cu) - 1) if cu[b] <= t)


def test_planted_violations(mods):
    L, wl = mods
    C = L.CHECK_CODES
    w = wl.ragged_prefill(device="cuda", n_req=6, e_lo=20, e_hi=90, c_lo=0, c_hi=70, num_slots=4096)
    base = _meta(w)
    rows, stride = base["page_table"].shape
    ns = base["num_slots"]
    tix = base["table_idx"].tolist()
    L_ = base["seq_lens"].tolist()
    Cl = base["cached_lens"].tolist()
    cu = base["cu_q"].tolist()

    def mut(field, idx, value):
        def f(m):
            t = m[field].clone()
            t[idx] = value
            m[field] = t
        return f

    def set_row(b, j, value):
        def f(m):
            t = m["page_table"].clone()
            t[tix[b], j] = value
            m["page_table"] = t
        return f

    def repeat(m):  # request 2's first new token takes request 0's first new slot, in the table and in out_loc
        s = int(m["out_loc"][cu[0]])
        pt = m["page_table"].clone()
        pt[tix[2], Cl[2]] = s
        m["page_table"] = pt
        loc = m["out_loc"].clone()
        loc[cu[2]] = s
        m["out_loc"] = loc

    def short_out_loc(m):
        m["out_loc"] = m["out_loc"][:-1].clone()

    t5 = 5
    used = set()
    for b in range(len(tix)):
        used.update(base["page_table"][tix[b], :L_[b]].tolist())
    other = next(x for x in range(ns) if x not in used and x != base["dummy_slot"])  # a slot no request uses
    cases = [
        ("table_idx past the rows", mut("table_idx", 2, rows), "table_idx", 2, None),
        ("negative table_idx", mut("table_idx", 1, -1), "table_idx", 1, None),
        ("zero seq_len", mut("seq_lens", 3, 0), "seq_len", 3, None),
        ("seq_len past the row", mut("seq_lens", 0, stride + 1), "seq_len", 0, None),
        ("cached_len = seq_len", mut("cached_lens", 4, L_[4]), "cached_len", 4, None),
        ("cu_q step", mut("cu_q", 2, cu[2] + 1), "cu_q", 1, None),
        ("cu_q[0] != 0", mut("cu_q", 0, 1), "cu_q", 0, None),
        ("slot past the pool", set_row(1, 3, ns), "slot", 1, None),
        ("negative slot", set_row(5, 0, -7), "slot", 5, None),
        ("out_loc not the row's entry", mut("out_loc", t5, other), "out_loc", _token_owner(base, t5), t5),
        ("out_loc past the pool", mut("out_loc", t5, ns + 3), "out_loc", _token_owner(base, t5), t5),
        ("repeated new slot", repeat, "repeat", None, None),
        ("out_loc one short", short_out_loc, "token_count", 5, None),
    ]
    for name, f, code, first_req, first_tok in cases:
        m = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
        f(m)
        r, host_ok = _run(L, m)
        say(f"[check] {name}: {r} host_ok={host_ok}")
        assert not host_ok, name
        assert r[0] & C[code], (name, r)
        assert r[1] >= 1, (name, r)
        if first_req is not None:
            assert r[2] == first_req, (name, r)
        else:  # a repeat is recorded by whichever of the two tokens comes second (atomic order)
            assert r[1] == 1 and r[2] in (0, 2) and r[3] in (cu[0], cu[2]), (name, r)
        if first_tok is not None:
            assert r[3] == first_tok, (name, r)
    # pages: page size 16 decode batch
    d = wl.qwen3_8b_decode(page_size=16, bs=7, num_slots=1 << 12, median=100.0, hi=512, device="cuda")
    dm = _meta(d)
    b = int(np.argmax(dm["seq_lens"].numpy() > 33))
    assert int(dm["seq_lens"][b]) > 33
    row = int(dm["table_idx"][b])
    for j, name in ((17, "slot inside a page"), (16, "page start not a multiple of 16")):
        m = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in dm.items()}
        pt = m["page_table"].clone()
        pt[row, j] += 1
        m["page_table"] = pt
        r, host_ok = _run(L, m)
        say(f"[check] {name}: {r} host_ok={host_ok}")
        assert not host_ok and r[0] & C["page"] and r[2] == b, (name, r)


def test_random_corruptions_agree_with_host(mods):
    L, wl = mods
    w = wl.ragged_prefill(device="cuda", n_req=6, e_lo=20, e_hi=90, c_lo=0, c_hi=70, num_slots=4096)
    d = wl.qwen3_8b_decode(page_size=16, bs=7, num_slots=1 << 12, median=100.0, hi=512, device="cuda")
    rng = np.random.default_rng(77)
    agree = flagged = 0
    for base in (_meta(w), _meta(d)):
        for it in range(60):
            m = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in base.items()}
            for _ in range(int(rng.integers(1, 3))):
                field = ["page_table", "table_idx", "seq_lens", "cached_lens", "cu_q", "out_loc"][int(rng.integers(6))]
                t = m[field].view(-1)
                i = int(rng.integers(t.numel()))
                v = int(t[i])
                t[i] = int(rng.choice([v + 1, v - 1, -1, 0, 2 ** 31 - 1, -2 ** 31, v + 16, int(rng.integers(-5, 5000))]))
            r, host_ok = _run(L, m)
            assert (r[0] == 0) == host_ok, (it, r, host_ok)
            assert (r[0] == 0) == (r[1] == 0 and r[2] == INT_MAX), r
            agree += 1
            flagged += r[0] != 0
    say(f"[check] random corruptions: {agree} agree with the host validator, {flagged} flagged")
    assert flagged >= agree // 4


def test_check_batch_under_graph_capture(mods):
    """The check records into a captured graph (kernels only, no memset) and
    each replay re-checks whatever the recorded buffers hold."""
    L, wl = mods
    w = wl.ragged_prefill(device="cuda", n_req=6, e_lo=20, e_hi=90, c_lo=0, c_hi=70, num_slots=4096)
    m = _meta(w)
    g_ = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in m.items()}
    result = torch.empty(4, dtype=torch.int32, device="cuda")
    seen = torch.empty((m["num_slots"] + 31) // 32, dtype=torch.int32, device="cuda")
    st = torch.cuda.Stream()
    call = lambda: L.msgl_check_batch(g_["page_table"], g_["table_idx"], g_["seq_lens"], g_["cached_lens"],
                                      g_["cu_q"], m["max_seq_len"], m["num_slots"], m["page_size"],
                                      out_loc=g_["out_loc"], dummy_slot=m["dummy_slot"], result=result, seen=seen,
                                      stream=st)
    with torch.cuda.stream(st):
        call()  # eager once before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        call()
    torch.cuda.synchronize()
    good = list(g_["seq_lens"].cpu())
    for rnd in range(3):
        result.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        assert [int(x) for x in result.cpu()] == [0, 0, INT_MAX, INT_MAX], rnd
        g_["seq_lens"][2] = 0  # a violation planted in the recorded buffer
        graph.replay()
        torch.cuda.synchronize()
        r = [int(x) for x in result.cpu()]
        assert r[0] & L.CHECK_CODES["seq_len"] and r[2] == 2, (rnd, r)
        g_["seq_lens"][2] = int(good[2])
