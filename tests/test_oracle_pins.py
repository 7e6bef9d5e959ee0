"""Pins of the fp64 oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a wrong kv-head index, a wrong causal offset, a transposed
operand, a missing max subtraction) fails at least one of them:

* brute force in pure Python lists (``math.exp`` / ``math.fsum``) over the full
  score matrix on the tiny workload, decode and prefill;
* a textbook dense routine (``torch.nn.functional.scaled_dot_product_attention``
  in fp64 with an explicit bottom-right causal mask) on an identity page table;
* closed forms: a length-1 context returns V; identical keys give the mean of
  the visible V rows; V = 1 gives exactly 1;
* invariants: permuting pool slots together with the page table, page size 1
  versus 16 on the same logical K/V, a constant added to every logit,
  GQA versus MHA with repeated K/V, a decode row versus the last prefill row,
  an extend with a cached prefix versus the tail rows of a full prefill, and
  softmax row sums from ``lse``;
* store_kv: written rows equal the new rows, every other slot is unchanged.
"""

import cmath
import math

import numpy as np
import pytest
import torch

from paged_kv_attention_slots_amd import workloads as wl


def _f64(t):
    return t.to(torch.float64)


def _brute(w, kp, vp):
    """Pure-Python attention straight from the definition: gather, full score
    matrix, mask, softmax with max subtraction, weighted sum."""
    H, G, d = w.q_heads, w.kv_heads, w.head_dim
    g = H // G
    scale = 1.0 / math.sqrt(d)
    q = _f64(w.q).tolist()
    K = _f64(kp).tolist()
    V = _f64(vp).tolist()
    pt = w.page_table.tolist()
    out = [[None] * H for _ in range(w.num_tokens)]
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        c0, c1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        n = c1 - c0
        row = pt[int(w.table_idx[b])]
        for i in range(n):
            p = L - n + i
            for h in range(H):
                kv = h // g
                scores = []
                for j in range(L):  # full row, then mask
                    kj = K[row[j]][kv]
                    scores.append(scale * math.fsum(a * b_ for a, b_ in zip(q[c0 + i][h], kj)))
                vis = [s for j, s in enumerate(scores) if j <= p]
                m = max(vis)
                e = [math.exp(s - m) for s in vis]
                l = math.fsum(e)
                o = [math.fsum(e[j] * V[row[j]][kv][c] for j in range(p + 1)) / l for c in range(d)]
                out[c0 + i][h] = o
    return torch.tensor(out, dtype=torch.float64)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_bruteforce_tiny(oracle_mod, mode):
    w = wl.tiny(mode)
    kp, vp, out, lse = oracle_mod.step(w)
    ref = _brute(w, kp, vp)
    assert out.shape == ref.shape
    assert torch.max(torch.abs(out - ref)).item() < 1e-12


def _identity_workload(lens, cached, H, G, d, seed=7, dtype=torch.float32):
    S = int(sum(lens)) + 64
    rows, pos = [], 0
    for L in lens:
        rows.append(np.arange(pos, pos + L))
        pos += L
    return wl.build_workload("ident", "prefill", dtype, H, G, d, 1, S, len(lens), max(lens),
                             rows, lens, cached, seed)


def test_sdpa_contiguous(oracle_mod):
    lens = [37, 70, 129]
    cached = [0, 25, 64]
    w = _identity_workload(lens, cached, H=8, G=2, d=64)
    kp, vp, out, _ = oracle_mod.step(w)
    g = w.q_heads // w.kv_heads
    for b, (L, C) in enumerate(zip(lens, cached)):
        row = w.page_table[b, :L].long()
        K = _f64(kp[row]).repeat_interleave(g, dim=1).transpose(0, 1)  # [H, L, d]
        V = _f64(vp[row]).repeat_interleave(g, dim=1).transpose(0, 1)
        c0, c1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        Q = _f64(w.q[c0:c1]).transpose(0, 1)  # [H, n, d]
        n = c1 - c0
        pos = torch.arange(C, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos  # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K.contiguous(), V.contiguous(),
                                                               attn_mask=mask)
        assert n == L - C
        err = torch.max(torch.abs(out[c0:c1] - ref.transpose(0, 1))).item()
        assert err < 1e-12, (b, err)


def test_length_one_returns_v(oracle_mod):
    w = _identity_workload([1, 1, 3], [0, 0, 2], H=4, G=2, d=64)
    kp, vp, out, lse = oracle_mod.step(w)
    g = 2
    for b in range(2):
        slot = int(w.page_table[b, 0])
        for h in range(4):
            assert torch.equal(out[b, h], _f64(vp[slot, h // g]))
            s = (_f64(w.q[b, h]) * _f64(kp[slot, h // g])).sum().item() / 8.0
            assert abs(lse[b, h].item() - s) < 1e-12


def test_identical_keys_give_mean_of_v(oracle_mod):
    w = _identity_workload([11, 20], [0, 5], H=4, G=2, d=64)
    kp, vp, _, _ = oracle_mod.step(w)
    kp[:] = kp[0:1]  # every slot holds the same key
    out, _ = oracle_mod.attention(w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        c0, c1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        for i in range(c1 - c0):
            p = L - (c1 - c0) + i
            rows = w.page_table[b, :p + 1].long()
            for h in range(4):
                mean = [math.fsum(x) / (p + 1) for x in _f64(vp[rows, h // 2]).T.tolist()]
                assert torch.max(torch.abs(out[c0 + i, h] - torch.tensor(mean, dtype=torch.float64))) < 1e-12


def test_v_ones_gives_exactly_one(oracle_mod):
    w = wl.tiny("prefill")
    kp, vp = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    out, _ = oracle_mod.attention(w.q, kp, torch.ones_like(vp), w.page_table, w.table_idx,
                                  w.seq_lens, w.cu_q)
    assert torch.equal(out, torch.ones_like(out))


def test_permuting_slots_with_table(oracle_mod):
    w = wl.tiny("prefill")
    kp, vp, out, lse = oracle_mod.step(w)
    S = kp.shape[0]
    perm = torch.from_numpy(np.random.default_rng(3).permutation(S))
    kp2 = torch.empty_like(kp)
    vp2 = torch.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    pt2 = perm[w.page_table.long()].to(torch.int32)
    out2, lse2 = oracle_mod.attention(w.q, kp2, vp2, pt2, w.table_idx, w.seq_lens, w.cu_q)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_page_size_invariance(oracle_mod):
    kw = dict(bs=5, num_slots=1 << 13, median=300.0, hi=1024,
              heads=dict(H=8, G=2, d=64))
    w1 = wl.qwen3_8b_decode(page_size=1, **kw)
    w16 = wl.qwen3_8b_decode(page_size=16, **kw)
    assert torch.equal(w1.seq_lens, w16.seq_lens)
    assert not torch.equal(w1.page_table[:5, :100], w16.page_table[:5, :100])
    _, _, o1, l1 = oracle_mod.step(w1)
    _, _, o16, l16 = oracle_mod.step(w16)
    assert torch.equal(o1, o16) and torch.equal(l1, l16)


def test_logit_shift_invariance(oracle_mod):
    # keys all carry the same value in the last dim; moving q's last component
    # adds the same constant (here +800, beyond exp's double range) to every
    # logit of that head, which the max subtraction must absorb
    w = _identity_workload([9, 33], [0, 10], H=4, G=2, d=64)
    kp, vp = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    kp[:, :, -1] = 2.0
    q0 = w.q.clone()
    q0[:, :, -1] = 0.0
    q1 = q0.clone()
    q1[:, :, -1] = 800.0 * 8.0 / 2.0  # scale 1/8 -> shift of exactly 800
    o0, l0 = oracle_mod.attention(q0, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    o1, l1 = oracle_mod.attention(q1, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    assert torch.isfinite(o1).all()
    assert torch.max(torch.abs(o0 - o1)).item() < 1e-9
    assert torch.max(torch.abs((l1 - 800.0) - l0)).item() < 1e-9


def test_gqa_equals_mha_with_repeated_kv(oracle_mod):
    w = _identity_workload([17, 40], [3, 0], H=8, G=2, d=64)
    kp, vp = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    o_gqa, _ = oracle_mod.attention(w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    kp_m = kp.repeat_interleave(4, dim=1).contiguous()
    vp_m = vp.repeat_interleave(4, dim=1).contiguous()
    o_mha, _ = oracle_mod.attention(w.q, kp_m, vp_m, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    assert torch.equal(o_gqa, o_mha)
    # and a wrong grouping (h % G) would differ
    kp_w = kp.repeat(1, 4, 1).contiguous()
    vp_w = vp.repeat(1, 4, 1).contiguous()
    o_w, _ = oracle_mod.attention(w.q, kp_w, vp_w, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
    assert not torch.allclose(o_gqa, o_w)


def test_decode_row_is_last_prefill_row(oracle_mod):
    wp = wl.tiny("prefill")
    wd = wl.tiny("decode")
    _, _, op, lp = oracle_mod.step(wp)
    _, _, od, ld = oracle_mod.step(wd)
    # decode q is drawn for its own step; re-run decode with the prefill rows' q
    kp, vp = oracle_mod.store_kv(wp.k_pool, wp.v_pool, wp.k_new, wp.v_new, wp.out_loc)
    last = (wp.cu_q[1:] - 1).long()
    od2, ld2 = oracle_mod.attention(wp.q[last], kp, vp, wp.page_table, wp.table_idx, wp.seq_lens,
                                    torch.arange(wp.bs + 1, dtype=torch.int32))
    assert torch.equal(od2, op[last]) and torch.equal(ld2, lp[last])
    # the decode workload's pool after store_kv equals the prefill one on live rows
    kpd, vpd = oracle_mod.store_kv(wd.k_pool, wd.v_pool, wd.k_new, wd.v_new, wd.out_loc)
    for b in range(wd.bs):
        row = wd.page_table[b, :int(wd.seq_lens[b])].long()
        assert torch.equal(kpd[row], kp[row]) and torch.equal(vpd[row], vp[row])


def test_extend_equals_tail_of_full_prefill(oracle_mod):
    lens = [30, 45]
    full = _identity_workload(lens, [0, 0], H=4, G=2, d=64)
    kp, vp, of, lf = oracle_mod.step(full)
    cached = [12, 40]
    cu = torch.tensor([0, lens[0] - cached[0], lens[0] - cached[0] + lens[1] - cached[1]],
                      dtype=torch.int32)
    rows_q = torch.cat([torch.arange(cached[0], lens[0]), lens[0] + torch.arange(cached[1], lens[1])])
    oe, le = oracle_mod.attention(full.q[rows_q], kp, vp, full.page_table, full.table_idx,
                                  full.seq_lens, cu)
    assert torch.equal(oe, of[rows_q]) and torch.equal(le, lf[rows_q])


def test_row_sums_from_lse(oracle_mod):
    w = wl.tiny("prefill")
    kp, vp, out, lse = oracle_mod.step(w)
    for b in range(w.bs):
        L = int(w.seq_lens[b])
        row = w.page_table[b, :L].long()
        c0, c1 = int(w.cu_q[b]), int(w.cu_q[b + 1])
        for i in range(c1 - c0):
            p = L - (c1 - c0) + i
            for h in range(w.q_heads):
                K = _f64(kp[row[:p + 1], h // 2]).numpy()
                s = K @ _f64(w.q[c0 + i, h]).numpy() / 8.0
                tot = math.fsum(np.exp(s - lse[c0 + i, h].item()).tolist())
                assert abs(tot - 1.0) < 1e-12


def test_store_kv_definition(oracle_mod):
    w = wl.qwen3_06b_decode(bs=6, lo=20, hi=60, num_slots=1 << 10)
    kp, vp = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    loc = w.out_loc.long()
    assert torch.equal(kp[loc].view(torch.int16), w.k_new.view(torch.int16))
    assert torch.equal(vp[loc].view(torch.int16), w.v_new.view(torch.int16))
    untouched = torch.ones(kp.shape[0], dtype=torch.bool)
    untouched[loc] = False
    assert torch.equal(kp[untouched].view(torch.int16), w.k_pool[untouched].view(torch.int16))
    assert torch.equal(vp[untouched].view(torch.int16), w.v_pool[untouched].view(torch.int16))
    # inputs untouched
    assert not torch.equal(kp.view(torch.int16), w.k_pool.view(torch.int16))


def test_bf16_widening_is_exact(oracle_mod):
    # one key, one value: the output must be the bf16 value widened exactly
    x = torch.tensor([1.0 + 2 ** -7, -3.5, 2 ** -120, 65280.0], dtype=torch.bfloat16)
    H, G, d = 1, 1, 64
    kp = torch.zeros(2, G, d, dtype=torch.bfloat16)
    vp = torch.zeros(2, G, d, dtype=torch.bfloat16)
    vp[1, 0, :4] = x
    q = torch.zeros(1, H, d, dtype=torch.bfloat16)
    pt = torch.tensor([[1] * 32], dtype=torch.int32)
    out, lse = oracle_mod.attention(q, kp, vp, pt, torch.tensor([0], dtype=torch.int32),
                                    torch.tensor([1], dtype=torch.int32),
                                    torch.tensor([0, 1], dtype=torch.int32))
    assert out[0, 0, :4].tolist() == [1.0 + 2 ** -7, -3.5, 2 ** -120, 65280.0]
    assert lse[0, 0].item() == 0.0


# ---------------------------------------------------------------------------
# Rotary embedding (the step before the KV write in the layer's pipeline).
# Pins: position 0 is the identity; with two dimensions the embedding is the
# complex rotation (x0 + i x1) e^{ip}; with four dimensions and base 10^4 the
# two pairs turn by p and p / 100 (angles worked out by hand); every pair
# keeps its length; q.k depends only on the distance between positions.

def _rope_inputs(T=6, heads=3, d=8, seed=7, dtype=torch.float32, max_pos=40000):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, heads, d, generator=g).to(dtype)
    pos = torch.randint(0, max_pos, (T,), generator=g, dtype=torch.int32)
    return x, pos


def test_rope_position_zero_is_identity(oracle_mod):
    x, _ = _rope_inputs(dtype=torch.bfloat16, d=128)
    out = oracle_mod.rope(x, torch.zeros(x.shape[0], dtype=torch.int32), 1e6)
    assert torch.equal(out, x.double())


def test_rope_two_dims_is_complex_rotation(oracle_mod):
    x, pos = _rope_inputs(d=2)
    out = oracle_mod.rope(x, pos, 12345.0)  # the only frequency is base**0 = 1
    for t in range(x.shape[0]):
        for h in range(x.shape[1]):
            z = complex(float(x[t, h, 0]), float(x[t, h, 1])) * cmath.exp(1j * int(pos[t]))
            assert abs(float(out[t, h, 0]) - z.real) < 1e-12
            assert abs(float(out[t, h, 1]) - z.imag) < 1e-12


def test_rope_four_dims_frequencies(oracle_mod):
    # d = 4, base = 10^4: elements (0, 2) turn by p radians, (1, 3) by p / 100
    x, _ = _rope_inputs(T=5, heads=2, d=4)
    pos = torch.tensor([0, 1, 2, 50, 314], dtype=torch.int32)
    out = oracle_mod.rope(x, pos, 1e4)
    for t in range(5):
        p = int(pos[t])
        for h in range(2):
            for i, angle in ((0, float(p)), (1, p / 100.0)):
                z = complex(float(x[t, h, i]), float(x[t, h, i + 2])) * cmath.exp(1j * angle)
                assert abs(float(out[t, h, i]) - z.real) < 1e-12, (t, h, i)
                assert abs(float(out[t, h, i + 2]) - z.imag) < 1e-12, (t, h, i)


def test_rope_keeps_pair_lengths(oracle_mod):
    x, pos = _rope_inputs(T=16, heads=4, d=128, dtype=torch.bfloat16)
    out = oracle_mod.rope(x, pos, 1e6)
    xd = x.double()
    n_in = xd[..., :64] ** 2 + xd[..., 64:] ** 2
    n_out = out[..., :64] ** 2 + out[..., 64:] ** 2
    assert torch.allclose(n_out, n_in, rtol=1e-12, atol=1e-14)
    assert not torch.allclose(out, xd)


def test_rope_scores_depend_on_distance_only(oracle_mod):
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, 1, 64, generator=g, dtype=torch.float32)
    k = torch.randn(1, 1, 64, generator=g, dtype=torch.float32)

    def score(m, n):
        rq = oracle_mod.rope(q, torch.tensor([m], dtype=torch.int32), 1e4)
        rk = oracle_mod.rope(k, torch.tensor([n], dtype=torch.int32), 1e4)
        return float((rq * rk).sum())

    bound = 1e-9 * float(q.double().norm() * k.double().norm())
    for m, n in ((7, 3), (3, 7), (100, 0), (5, 5)):
        ref = score(m, n)
        for shift in (1, 17, 1000, 30000):
            assert abs(score(m + shift, n + shift) - ref) < bound, (m, n, shift)
    assert abs(score(5, 5) - float((q.double() * k.double()).sum())) < bound
    assert abs(score(7, 3) - score(3, 7)) > 1e-3  # the sign of the distance matters


def test_rope_store_kv_definition(oracle_mod):
    g = torch.Generator().manual_seed(3)
    T, H, G, d, S = 5, 4, 2, 64, 32
    q = torch.randn(T, H, d, generator=g).to(torch.bfloat16)
    k = torch.randn(T, G, d, generator=g).to(torch.bfloat16)
    v = torch.randn(T, G, d, generator=g).to(torch.bfloat16)
    vp = torch.randn(S, G, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([0, 9, 4, 31, 2], dtype=torch.int32)
    loc = torch.tensor([3, 17, 0, 31, 8], dtype=torch.int32)
    q_rot, k_rot, vp2 = oracle_mod.rope_store_kv(q, k, v, vp, pos, loc, 1e6)
    assert torch.equal(q_rot, oracle_mod.rope(q, pos, 1e6))
    assert torch.equal(k_rot, oracle_mod.rope(k, pos, 1e6))
    assert torch.equal(q_rot[0], q[0].double()) and torch.equal(k_rot[0], k[0].double())
    assert torch.equal(vp2[loc.long()].view(torch.int16), v.view(torch.int16))
    untouched = torch.ones(S, dtype=torch.bool)
    untouched[loc.long()] = False
    assert torch.equal(vp2[untouched].view(torch.int16), vp[untouched].view(torch.int16))


# --------------------------------------------------------------------------
# vocabulary indexing (the embedding rows of the step's token ids, sharded by
# vocabulary range as under tensor parallelism)
# --------------------------------------------------------------------------


def test_vocab_embed_hand_worked(oracle_mod):
    # a shard holding ids 2..5 of the vocabulary: rows 10*r + (0, 1)
    # (a view of a larger table: the row after the shard is real memory, so a
    # range check that lets id 6 through reads 99s rather than garbage)
    w = torch.tensor([[0.0, 1.0], [10.0, 11.0], [20.0, 21.0], [30.0, 31.0], [99.0, 99.0]])[:4]
    ids = torch.tensor([1, 2, 3, 5, 6, -1, 4], dtype=torch.int32)
    out = oracle_mod.vocab_embed(w, ids, vocab_start=2)
    expect = torch.tensor([[0.0, 0.0], [0.0, 1.0], [10.0, 11.0], [30.0, 31.0], [0.0, 0.0], [0.0, 0.0],
                           [20.0, 21.0]])
    assert torch.equal(out, expect)


def test_vocab_embed_full_table_is_embedding(oracle_mod):
    g = torch.Generator().manual_seed(21)
    w = torch.randn(1000, 64, generator=g).to(torch.bfloat16)
    ids = torch.randint(0, 1000, (300,), generator=g, dtype=torch.int32)
    out = oracle_mod.vocab_embed(w, ids)
    ref = torch.nn.functional.embedding(ids.long(), w)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("shards", [2, 3, 4])
def test_vocab_embed_shards_sum_to_full_table(oracle_mod, shards):
    """Tensor-parallel split of the vocabulary: exactly one shard holds each
    id, so the shards' outputs are the full rows there and zero elsewhere,
    and they sum (all-reduce) to the full table's rows."""
    g = torch.Generator().manual_seed(22)
    V, hid = 997, 32
    w = torch.randn(V, hid, generator=g)
    bounds = [V * i // shards for i in range(shards + 1)]
    edges = [x for i in range(shards) for x in (bounds[i], bounds[i + 1] - 1)]  # each shard's first and last id
    ids = torch.cat([torch.randint(0, V, (257,), generator=g, dtype=torch.int32),
                     torch.tensor(edges, dtype=torch.int32)])
    full = oracle_mod.vocab_embed(w, ids)
    total = torch.zeros_like(full, dtype=torch.float64)
    owners = torch.zeros(ids.numel(), dtype=torch.int64)
    for i in range(shards):
        part = oracle_mod.vocab_embed(w[bounds[i]:bounds[i + 1]], ids, vocab_start=bounds[i])
        nz = (part != 0).any(dim=1)
        owners += nz.long()
        total += part.double()
    assert torch.equal(total, full.double())
    assert bool((owners == 1).all())  # randn rows have no all-zero row
