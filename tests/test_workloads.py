"""Host-side input generation: determinism, page-table structure, metadata,
and the layout / sizing figures the pages print (tests/golden/page_figures.json)."""

import json
import os

import numpy as np
import pytest
import torch

from paged_kv_attention_slots_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_pool_and_table_shapes():
    g = _golden()
    for c in g["pool_shape"]:
        assert list(wl.pool_shape(c["num_pages"], c["page_size"], c["kv_heads"], c["head_dim"])) == c["shape"]
    for c in g["page_table_shape"]:
        assert list(wl.page_table_shape(c["max_running_req"], c["max_seq_len"])) == c["shape"]


def test_golden_kv_sizing():
    g = _golden()
    for c in g["kv_bytes_per_token"]:
        assert wl.kv_bytes_per_token(c["head_dim"], c["kv_heads"], c["itemsize"], c["num_layers"]) == c["bytes"]
    c = g["kv_capacity_tokens"][0]
    per = wl.kv_bytes_per_token(128, 8, 2, 28)
    usable = c["memory_ratio"] * c["card_bytes"] - c["model_bytes"]
    assert abs(usable / per - c["approx_tokens"]) / c["approx_tokens"] < c["rel_tol"]


def test_golden_graph_padding():
    c = _golden()["graph_padding"][0]
    assert wl.padded_batch_size(c["bs"], c["recorded"]) == c["padded"]
    assert wl.padded_batch_size(100) == 128 and wl.padded_batch_size(256) == 256
    with pytest.raises(ValueError):
        wl.padded_batch_size(257)


def test_hash_generator_is_chunk_independent():
    a = wl.gen_values(5, 1, 1000, 5000, 1.0, torch.bfloat16, "cpu", chunk=777)
    b = wl.gen_values(5, 1, 1000, 5000, 1.0, torch.bfloat16, "cpu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rows = wl.gen_rows(5, 1, torch.arange(1, 6), 1000, 1.0, torch.bfloat16, "cpu")
    assert torch.equal(rows.reshape(-1).view(torch.int16), b.view(torch.int16))
    # large indices (beyond 2**32) still hash, and differ from small ones
    big = wl.gen_values(5, 1, (1 << 33) + 1000, 5000, 1.0, torch.bfloat16, "cpu")
    assert not torch.equal(big.view(torch.int16), b.view(torch.int16))


def test_hash_generator_distribution():
    x = wl.gen_values(11, 2, 0, 1 << 20, 1.0, torch.float32, "cpu").double()
    assert abs(x.mean().item()) < 0.01 and abs(x.std().item() - 1.0) < 0.01
    y = wl.gen_values(11, 3, 0, 1 << 20, 1.0 / np.sqrt(128), torch.bfloat16, "cpu").double()
    assert abs(y.std().item() - 1.0 / np.sqrt(128)) < 0.002
    # bf16 table entries are exactly representable
    t = wl.normal_table(1.0, torch.bfloat16)
    assert torch.equal(t, t.to(torch.bfloat16).to(torch.float32))


def test_determinism():
    a = wl.qwen3_06b_decode(bs=4, lo=16, hi=64, num_slots=1 << 10)
    b = wl.qwen3_06b_decode(bs=4, lo=16, hi=64, num_slots=1 << 10)
    for name in ("page_table", "seq_lens", "out_loc", "positions", "cu_q"):
        assert torch.equal(getattr(a, name), getattr(b, name))
    for name in ("k_pool", "v_pool", "k_new", "v_new", "q"):
        assert torch.equal(getattr(a, name).view(torch.int16), getattr(b, name).view(torch.int16))


def _check_structure(w):
    pt = w.page_table
    R = w.max_running_req
    assert pt.dtype == torch.int32 and pt.shape[1] % 32 == 0 and pt.shape[0] == R + 1
    assert torch.all(pt[R] == w.dummy_slot)
    live = []
    for b in range(w.bs):
        L, C = int(w.seq_lens[b]), int(w.cached_lens[b])
        assert 0 <= C < L <= pt.shape[1]
        row = pt[int(w.table_idx[b]), :L]
        assert int(row.min()) >= 0 and int(row.max()) < w.num_slots
        live.append(row)
    live = torch.cat(live)
    assert torch.unique(live).numel() == live.numel(), "live slots alias"
    ext = w.seq_lens - w.cached_lens
    assert torch.equal(w.cu_q[1:] - w.cu_q[:-1], ext)
    t = 0
    for b in range(w.bs):
        L, C = int(w.seq_lens[b]), int(w.cached_lens[b])
        assert torch.equal(w.positions[t:t + L - C], torch.arange(C, L, dtype=torch.int32))
        assert torch.equal(w.out_loc[t:t + L - C], pt[int(w.table_idx[b]), C:L])
        t += L - C
    assert w.q.shape == (t, w.q_heads, w.head_dim)
    assert w.k_new.shape == (t, w.kv_heads, w.head_dim)
    assert w.k_pool.shape == (w.num_slots + w.page_size, w.kv_heads, w.head_dim)


def test_structure_all_configs_small():
    _check_structure(wl.tiny("decode"))
    _check_structure(wl.tiny("prefill"))
    _check_structure(wl.qwen3_06b_decode(bs=8, lo=16, hi=200, num_slots=1 << 12))
    _check_structure(wl.ragged_prefill(n_req=3, e_lo=8, e_hi=40, c_hi=30, num_slots=1 << 9))
    _check_structure(wl.qwen3_8b_decode(page_size=1, bs=6, num_slots=1 << 14, median=200.0, hi=2048))
    _check_structure(wl.qwen3_8b_decode(page_size=16, bs=6, num_slots=1 << 14, median=200.0, hi=2048))


def test_tiny_rows_are_permutations():
    w = wl.tiny("decode")
    for b in range(2):
        row = w.page_table[b].numpy()
        assert sorted(row.tolist()) == list(range(256))


def test_page_size_16_rows_are_page_contiguous():
    w = wl.qwen3_8b_decode(page_size=16, bs=6, num_slots=1 << 14, median=200.0, hi=2048)
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        row = w.page_table[b, :L].long()
        j = torch.arange(L)
        first = row[(j // 16) * 16]
        assert torch.all(first % 16 == 0)
        assert torch.equal(row, first + j % 16)


def test_same_logical_kv_across_page_sizes():
    kw = dict(bs=4, num_slots=1 << 13, median=100.0, hi=1024)
    a = wl.qwen3_8b_decode(page_size=1, **kw)
    b = wl.qwen3_8b_decode(page_size=16, **kw)
    for r in range(4):
        L = int(a.seq_lens[r])
        ra = a.page_table[r, :L - 1].long()
        rb = b.page_table[r, :L - 1].long()
        assert torch.equal(a.k_pool[ra].view(torch.int16), b.k_pool[rb].view(torch.int16))
        assert torch.equal(a.v_pool[ra].view(torch.int16), b.v_pool[rb].view(torch.int16))
    assert torch.equal(a.k_new.view(torch.int16), b.k_new.view(torch.int16))
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))


def test_pad_decode_uses_dummy_row():
    w = wl.qwen3_06b_decode(bs=3, lo=16, hi=64, num_slots=1 << 10)
    p = wl.pad_decode(w, 4)
    assert p.bs == 4
    assert int(p.table_idx[3]) == w.max_running_req
    assert int(p.seq_lens[3]) == 1 and int(p.cached_lens[3]) == 0
    assert int(p.out_loc[3]) == w.dummy_slot
    assert int(p.page_table[int(p.table_idx[3]), 0]) == w.dummy_slot


def test_lognormal_lengths():
    rng = np.random.default_rng(0)
    L = wl.lognormal_lengths(rng, 200000)
    assert L.min() >= 16 and L.max() <= 32768
    assert abs(np.median(L) - 2048) / 2048 < 0.02


# --------------------------------------------------------------------------
# shared radix prefixes: generator structure and the host validator
# --------------------------------------------------------------------------


@pytest.mark.parametrize("page_size", [1, 16])
def test_shared_prefix_batch_structure(page_size):
    from paged_kv_attention_slots_amd import _lib as L

    sp = wl.shared_prefix_decode(group_sizes=(3, 2, 1), prefixes=(48, 16, 32), singles=2, suffix_hi=50,
                                 num_slots=4096, page_size=page_size)
    w = sp.w
    assert sp.group_start.tolist() == [0, 3, 5, 6]
    assert sp.prefix_lens.tolist() == [48, 48, 48, 16, 16, 32, 0, 0]
    pt = w.page_table
    for g in range(3):
        b0, b1 = int(sp.group_start[g]), int(sp.group_start[g + 1])
        P = int(sp.prefix_lens[b0])
        for b in range(b0, b1):
            assert torch.equal(pt[int(w.table_idx[b]), :P], pt[int(w.table_idx[b0]), :P])
    # slots outside the shared prefixes are used once
    used = torch.cat([pt[int(w.table_idx[b]), int(sp.prefix_lens[b]):int(w.seq_lens[b])] for b in range(w.bs)])
    assert used.unique().numel() == used.numel()
    L.msgl_validate_shared_prefix(pt, w.table_idx, w.seq_lens, sp.group_start, sp.prefix_lens, sp.max_group_size,
                                  sp.max_prefix_len)
    L.msgl_validate_batch(pt, w.table_idx, w.seq_lens, w.cached_lens, w.cu_q, max_seq_len=w.max_seq_len,
                          num_slots=w.num_slots, page_size=page_size, out_loc=w.out_loc, dummy_slot=w.dummy_slot)


def test_shared_prefix_validator_rejects():
    from paged_kv_attention_slots_amd import _lib as L

    sp = wl.shared_prefix_decode(group_sizes=(3, 2), prefixes=(48, 16), singles=1, suffix_hi=50, num_slots=4096)
    w = sp.w
    args = dict(max_group_size=sp.max_group_size, max_prefix_len=sp.max_prefix_len)

    def bad(pt=w.page_table, seq=w.seq_lens, gs=sp.group_start, pl=sp.prefix_lens, **kw):
        a = {**args, **kw}
        with pytest.raises(L.MsglError) as e:
            L.msgl_validate_shared_prefix(pt, w.table_idx, seq, gs, pl, a["max_group_size"], a["max_prefix_len"])
        return str(e.value)

    pt = w.page_table.clone()
    pt[int(w.table_idx[1]), 7] += 1
    assert "differs from its group's prefix" in bad(pt=pt)
    pl = sp.prefix_lens.clone()
    pl[2] = 40
    assert "differs from its group" in bad(pl=pl)
    seq = w.seq_lens.clone()
    seq[0] = 48  # the prefix would hold the new token
    assert "not in [0" in bad(seq=seq)
    gs = sp.group_start.clone()
    gs[0] = 1
    assert "group_start[0]" in bad(gs=gs)
    assert "max_group_size" in bad(max_group_size=2)
    assert "not in [0" in bad(max_prefix_len=20)
    pl = sp.prefix_lens.clone()
    pl[5] = 3  # the single request is in no group
    assert "in no group" in bad(pl=pl)


def test_validator_checks_out_loc_against_page_table():
    """out_loc must be page_table[row, cached:len] of each request in order:
    the captured decode step writes the new token's row where the request's
    last key is read."""
    from paged_kv_attention_slots_amd import _lib as L

    w = wl.qwen3_06b_decode(bs=6, lo=20, hi=60, num_slots=4096)
    args = dict(max_seq_len=w.max_seq_len, num_slots=w.num_slots, page_size=1, dummy_slot=w.dummy_slot)
    L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, None, None, out_loc=w.out_loc, **args)
    loc = w.out_loc.clone()
    loc[[1, 2]] = loc[[2, 1]]  # two requests' new slots swapped
    with pytest.raises(L.MsglError, match="expected page_table"):
        L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, None, None, out_loc=loc, **args)
    with pytest.raises(L.MsglError, match="entries"):
        L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, None, None, out_loc=w.out_loc[:4], **args)
    p = wl.ragged_prefill(n_req=3, e_lo=5, e_hi=20, c_hi=10, num_slots=1024)
    pargs = dict(max_seq_len=p.max_seq_len, num_slots=p.num_slots, page_size=1)
    L.msgl_validate_batch(p.page_table, p.table_idx, p.seq_lens, p.cached_lens, p.cu_q, out_loc=p.out_loc, **pargs)
    loc = p.out_loc.clone()
    loc[0] = loc[0] + 1 if int(loc[0]) + 1 < p.num_slots else loc[0] - 1
    with pytest.raises(L.MsglError, match="expected page_table"):
        L.msgl_validate_batch(p.page_table, p.table_idx, p.seq_lens, p.cached_lens, p.cu_q, out_loc=loc, **pargs)
