"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars: store_kv bit-exact on every slot but the dummy page's; attention
max-abs error <= 1e-5 for fp32 and <= 2e-2 for bf16 outputs; softmax row sums
from the returned lse within 1e-3 of 1.  Inputs are the seeded workloads;
the oracle gets host copies of the same inputs and computes store_kv itself.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import (ROWSUM_TOL, max_abs, oracle_rows, rowsum_error, sample_rows, say,
                            store_mismatch, tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def runner():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import runner as r

    return r


@pytest.fixture(scope="module")
def wl():
    from paged_kv_attention_slots_amd import workloads

    return workloads


def _full_check(oracle_mod, runner, w, chunk=0, rowsum_reqs=None):
    say(f"[parity] {w.name} bs={w.bs} T={w.num_tokens} H={w.q_heads} G={w.kv_heads} d={w.head_dim} "
        f"ps={w.page_size} chunk={chunk}")
    res = runner.run_step(w, chunk=chunk)
    torch.cuda.synchronize()
    kp, vp, out_ref, lse_ref = oracle_mod.step(w)
    assert store_mismatch(w, res.k_pool, res.v_pool, kp, vp) == 0
    err = max_abs(res.out, out_ref)
    say(f"[parity] {w.name}: max-abs {err:.3e}")
    assert err <= tol(w), err
    lse_err = max_abs(res.lse, lse_ref)
    assert lse_err < 1e-3, lse_err
    reqs = range(w.bs) if rowsum_reqs is None else rowsum_reqs
    rs = rowsum_error(w, kp, vp, res.lse, reqs)
    assert rs <= ROWSUM_TOL, rs
    return res, kp, vp, out_ref


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_fp32(oracle_mod, runner, wl, mode):
    w = wl.tiny(mode, device="cuda")
    _full_check(oracle_mod, runner, w)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_fp32_v_ones(oracle_mod, runner, wl, mode):
    w = wl.tiny(mode, device="cuda")
    w.v_pool.fill_(1.0)
    w.v_new.fill_(1.0)
    res = runner.run_step(w)
    assert max_abs(res.out, torch.ones(res.out.shape, dtype=torch.float64)) <= 1e-5


def test_qwen3_06b_decode(oracle_mod, runner, wl):
    w = wl.qwen3_06b_decode(device="cuda")
    _full_check(oracle_mod, runner, w)  # row sums of every request


def test_qwen3_06b_decode_v_ones_exact(runner, wl):
    w = wl.qwen3_06b_decode(device="cuda", bs=16)
    w.v_pool.fill_(1.0)
    w.v_new.fill_(1.0)
    res = runner.run_step(w)
    assert torch.equal(res.out.float().cpu(), torch.ones(res.out.shape))


@pytest.mark.parametrize("chunk", [64, 128, 1024])
def test_decode_chunk_sizes(oracle_mod, runner, wl, chunk):
    w = wl.qwen3_06b_decode(device="cuda", bs=24, seed=77)
    _full_check(oracle_mod, runner, w, chunk=chunk)


def test_qwen3_06b_decode_sharp_q(oracle_mod, runner, wl):
    # Q ~ N(0,1) makes the softmax peaked, so the bf16 bar discriminates
    w = wl.qwen3_06b_decode(device="cuda", q_std=1.0, seed=1012)
    _full_check(oracle_mod, runner, w)


@pytest.mark.parametrize("page_size", [1, 16])
def test_qwen3_8b_decode_full(oracle_mod, runner, wl, page_size):
    w = wl.qwen3_8b_decode(page_size=page_size, device="cuda")
    _full_check(oracle_mod, runner, w)  # row sums of every request


def test_qwen3_8b_decode_sharp_q(oracle_mod, runner, wl):
    w = wl.qwen3_8b_decode(page_size=16, device="cuda", bs=64, q_std=1.0, seed=1014)
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_small_full(oracle_mod, runner, wl):
    # every row, several tiles plus ragged tails, with and without a cached prefix
    w = wl.ragged_prefill(device="cuda", n_req=4, e_lo=1, e_hi=300, c_lo=0, c_hi=200, num_slots=1 << 12,
                          seed=31)
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_sharp_small(oracle_mod, runner, wl):
    w = wl.ragged_prefill(device="cuda", n_req=3, e_lo=60, e_hi=250, c_lo=0, c_hi=300, num_slots=1 << 12,
                          q_std=1.0, seed=32)
    _full_check(oracle_mod, runner, w)


@pytest.mark.parametrize("H,G", [(8, 8), (32, 8), (16, 2), (12, 3)])
def test_ragged_prefill_group_sizes(oracle_mod, runner, wl, H, G):
    # every supported grouping of q heads onto kv heads, with uneven tails
    w = wl.ragged_prefill(device="cuda", n_req=3, e_lo=1, e_hi=200, c_lo=0, c_hi=150, num_slots=1 << 11,
                          seed=40 + H + G, heads=dict(H=H, G=G, d=128))
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_long_prefix(oracle_mod, runner, wl):
    # a chunked-prefill shape: a long cached prefix, extends within and across key tiles
    w = wl.ragged_prefill(device="cuda", n_req=2, e_lo=100, e_hi=300, c_lo=2000, c_hi=3000,
                          num_slots=1 << 13, seed=45, heads=dict(H=32, G=8, d=128))
    _full_check(oracle_mod, runner, w)


@pytest.mark.parametrize("n_req", [100, 300])
def test_ragged_prefill_many_requests(oracle_mod, runner, wl, n_req):
    # more than 64 and more than 256 requests: the block enumeration keeps 4
    # or 16 requests per lane; short extends, some of one token
    w = wl.ragged_prefill(device="cuda", n_req=n_req, e_lo=1, e_hi=40, c_lo=0, c_hi=100,
                          num_slots=1 << 16, seed=50 + n_req)
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_page16(oracle_mod, runner, wl):
    # page size 16: the page table holds token-level slots of shuffled pages
    w = wl.ragged_prefill(device="cuda", n_req=4, e_lo=1, e_hi=300, c_lo=0, c_hi=400, num_slots=1 << 13,
                          seed=47, page_size=16)
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_beyond_mfma_batch(oracle_mod, runner, wl):
    # more requests than the matrix-core kernel takes (1024): the vector-ALU
    # kernel serves the call; sampled rows against the oracle
    w = wl.ragged_prefill(device="cuda", n_req=1030, e_lo=1, e_hi=6, c_lo=0, c_hi=60, num_slots=1 << 17,
                          seed=48)
    res = runner.run_step(w)
    torch.cuda.synchronize()
    kp, vp = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    assert store_mismatch(w, res.k_pool, res.v_pool, kp, vp) == 0
    rows = sample_rows(w, 256)
    out_ref, lse_ref = oracle_rows(oracle_mod, w, kp, vp, rows)
    idx = torch.from_numpy(rows).cuda()
    err = max_abs(res.out[idx], out_ref)
    say(f"[parity] prefill with {w.bs} requests, sampled {len(rows)} rows: max-abs {err:.3e}")
    assert err <= tol(w), err
    assert max_abs(res.lse[idx], lse_ref) < 1e-3


@pytest.mark.parametrize("H,G", [(16, 8), (32, 8)])
def test_ragged_prefill_long_chunks(oracle_mod, runner, wl, H, G):
    # 2048 or more new tokens per request: the single-block layout with the
    # deeper ring serves the call; every row against the oracle
    w = wl.ragged_prefill(device="cuda", n_req=2, e_lo=2048, e_hi=2300, c_lo=0, c_hi=300, num_slots=1 << 13,
                          seed=49 + H, heads=dict(H=H, G=G, d=128))
    assert w.num_tokens >= 2048 * w.bs
    _full_check(oracle_mod, runner, w)


def test_ragged_prefill_v_ones_exact(runner, wl):
    w = wl.ragged_prefill(device="cuda", n_req=3, e_lo=30, e_hi=300, c_lo=0, c_hi=200, num_slots=1 << 11,
                          seed=46)
    w.v_pool.fill_(1.0)
    w.v_new.fill_(1.0)
    res = runner.run_step(w)
    assert torch.equal(res.out.float().cpu(), torch.ones(res.out.shape))


def test_ragged_prefill_full_size_every_row(oracle_mod, runner, wl):
    # the ragged prefill batch at full size (8 requests, ~8k new tokens on
    # cached prefixes), every row and head against the oracle
    w = wl.ragged_prefill(device="cuda")
    say(f"[parity] {w.name} full size: T={w.num_tokens} lens={w.seq_lens.tolist()} "
        f"cached={w.cached_lens.tolist()}")
    _full_check(oracle_mod, runner, w)  # row sums of every query row and head


@pytest.mark.parametrize("e_lo,e_hi", [(30, 300), (2048, 2300)])
def test_ragged_prefill_v_ones_exact_sharp(runner, wl, e_lo, e_hi):
    # Q ~ N(0, 16): each row's softmax is dominated by a few keys, most often
    # past the first 32, whose weights are far from 1 and round to bf16 with
    # relative errors up to 2^-8.  With V = 1 the output is the applied
    # weights' sum over the normaliser, which must be exactly 1.  Both
    # matrix-core layouts (short extends, and 2048+ new tokens per request).
    w = wl.ragged_prefill(device="cuda", n_req=2, e_lo=e_lo, e_hi=e_hi, c_lo=0, c_hi=300, num_slots=1 << 13,
                          q_std=4.0, seed=60 + e_lo)
    w.v_pool.fill_(1.0)
    w.v_new.fill_(1.0)
    res = runner.run_step(w)
    o = res.out.float().cpu()
    bad = int((o != 1.0).sum())
    say(f"[parity] V=1 sharp prefill T={w.num_tokens}: {bad} outputs differ from 1 "
        f"(min {float(o.min()):.6f}, max {float(o.max()):.6f})")
    assert bad == 0


@pytest.mark.parametrize("heads,e_lo,e_hi", [(None, 1, 300), ("8b", 30, 700), (None, 2048, 2100)])
def test_prefill_without_lse_is_bit_identical(runner, wl, heads, e_lo, e_hi):
    # the kernels skip the unrounded weight sums when no lse is asked for; the
    # output (normalised by the rounded sums either way) must not change
    w = wl.ragged_prefill(device="cuda", n_req=3, e_lo=e_lo, e_hi=e_hi, c_lo=0, c_hi=400, num_slots=1 << 13,
                          seed=70 + e_lo, heads=wl.QWEN3_8B if heads == "8b" else wl.QWEN3_06B)
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    runner.store_kv(w, kp, vp)
    out_l, lse = runner.prefill_attn(w, kp, vp)
    out_n, none = runner.prefill_attn(w, kp, vp, with_lse=False)
    torch.cuda.synchronize()
    assert none is None and torch.isfinite(lse).all()
    assert torch.equal(out_n.view(torch.int16), out_l.view(torch.int16))


def test_length_one_returns_v_bitexact(runner, wl):
    w = wl.qwen3_8b_decode(page_size=1, device="cuda", bs=32, median=1.0, hi=1)
    assert int(w.seq_lens.max()) == 1
    w.seq_lens.fill_(1)
    res = runner.run_step(w)
    g = w.q_heads // w.kv_heads
    expect = w.v_new.repeat_interleave(g, dim=1)
    assert torch.equal(res.out.view(torch.int16), expect.view(torch.int16))


def test_permuting_slots_matches(runner, wl):
    w = wl.qwen3_06b_decode(device="cuda", bs=8, lo=100, hi=700, num_slots=1 << 13)
    res = runner.run_step(w, chunk=64)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.num_slots_total)).cuda()
    kp2 = torch.empty_like(w.k_pool)
    vp2 = torch.empty_like(w.v_pool)
    kp2[perm] = w.k_pool
    vp2[perm] = w.v_pool
    w2 = w.to("cuda")
    w2.k_pool, w2.v_pool = kp2, vp2
    w2.page_table = perm[w.page_table.long()].to(torch.int32)
    w2.out_loc = perm[w.out_loc.long()].to(torch.int32)
    res2 = runner.run_step(w2, chunk=64)
    # same summation order on the same values: bit-identical
    assert torch.equal(res.out.view(torch.int16), res2.out.view(torch.int16))


def test_padded_rows_do_not_disturb_real_rows(oracle_mod, runner, wl):
    w = wl.subset_decode(wl.qwen3_8b_decode(page_size=1, device="cuda", bs=8, median=600.0, hi=4096), 3)
    p = wl.pad_decode(w, 4)
    res = runner.run_step(p)
    torch.cuda.synchronize()
    _, _, out_ref, _ = oracle_mod.step(w)
    # the dummy request changes only where the key sequence is split between
    # blocks, hence rounding, never the value beyond the tolerance
    assert max_abs(res.out[:3], out_ref) <= 2e-2
    same = runner.run_step(p)
    assert torch.equal(res.out[:3].view(torch.int16), same.out[:3].view(torch.int16))


def test_empty_batch_is_noop(runner, wl):
    from paged_kv_attention_slots_amd import _lib

    w = wl.qwen3_06b_decode(device="cuda", bs=2, lo=10, hi=20, num_slots=256)
    ws = _lib.decode_workspace(0, w.q_heads, w.head_dim, w.max_seq_len)
    out = torch.empty_like(w.q[:0])
    _lib.msgl_decode_attn(out, None, w.q[:0], w.k_pool, w.v_pool, w.page_table, w.table_idx[:0],
                          w.seq_lens[:0], w.max_seq_len, ws)
    _lib.msgl_store_kv(w.k_pool, w.v_pool, w.k_new[:0], w.v_new[:0], w.out_loc[:0])
    torch.cuda.synchronize()
