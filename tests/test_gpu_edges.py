"""Edge cases of the attention step against the oracle: a request whose
history fills its whole page-table row (32768 keys, the longest context the
Qwen3-8B decode workload allows), one-key requests next to it, and prefill
requests with a single new token, with and without a cached prefix, beside
one that reaches the end of its row.  Bars as everywhere: store_kv bit-exact,
attention max-abs <= 2e-2 (bf16), lse within 1e-3, row sums within 1e-3."""

import numpy as np
import pytest
import torch

from tests.gpu_util import BF16_TOL, ROWSUM_TOL, max_abs, rowsum_error, say, store_mismatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import runner, workloads

    return runner, workloads


def _check(oracle_mod, runner, w):
    say(f"[edges] {w.name} lens={w.seq_lens.tolist()} cached={w.cached_lens.tolist()} ps={w.page_size}")
    res = runner.run_step(w)
    torch.cuda.synchronize()
    kp, vp, out_ref, lse_ref = oracle_mod.step(w)
    assert store_mismatch(w, res.k_pool, res.v_pool, kp, vp) == 0
    err = max_abs(res.out, out_ref)
    lse_err = max_abs(res.lse, lse_ref)
    rs = rowsum_error(w, kp, vp, res.lse, range(w.bs)) if w.num_tokens <= 300 else 0.0
    say(f"[edges] {w.name}: max-abs {err:.3e} lse {lse_err:.2e} rowsum {rs:.2e}")
    assert err <= BF16_TOL and lse_err < 1e-3 and rs <= ROWSUM_TOL, (err, lse_err, rs)


@pytest.mark.parametrize("page_size", [1, 16])
def test_decode_full_row_and_one_key(oracle_mod, mods, page_size):
    runner, wl = mods
    lens = [32768, 1, 2, 17, 4095]
    rng = np.random.default_rng(77)
    S = 1 << 17
    if page_size == 1:
        rows = wl.rows_from_free_slots(rng.permutation(S), lens)
    else:
        rows = wl.rows_from_free_pages(rng.permutation(S // page_size), lens, page_size)
    w = wl.build_workload(f"decode-edges-ps{page_size}", "decode", torch.bfloat16, **wl.QWEN3_8B,
                          page_size=page_size, num_slots=S, max_running_req=len(lens), max_seq_len=32768,
                          rows=rows, seq_lens=lens, cached_lens=[L - 1 for L in lens], seed=77, q_std=1.0,
                          device="cuda")
    assert w.row_stride == 32768
    _check(oracle_mod, runner, w)


def test_prefill_single_new_tokens_and_full_row(oracle_mod, mods):
    runner, wl = mods
    cached = [0, 5, 32700, 0, 63, 64]
    ext = [1, 1, 68, 130, 1, 65]
    lens = [c + e for c, e in zip(cached, ext)]
    rng = np.random.default_rng(78)
    rows = wl.rows_from_free_slots(rng.permutation(1 << 16), lens, new_after_history=False)
    w = wl.build_workload("prefill-edges", "prefill", torch.bfloat16, **wl.QWEN3_06B, page_size=1,
                          num_slots=1 << 16, max_running_req=len(lens), max_seq_len=32768, rows=rows,
                          seq_lens=lens, cached_lens=cached, seed=78, q_std=1.0, device="cuda")
    assert max(lens) == w.row_stride
    _check(oracle_mod, runner, w)


@pytest.mark.parametrize("chunk", [64, 128, 1024])
def test_decode_many_one_key_requests(oracle_mod, mods, chunk):
    """The decode split counts each request as its keys plus a fixed cost of
    work units; blocks whose share covers only a request's fixed-cost units
    must skip it, and the merge must find exactly the blocks holding its keys.
    A batch of one-key requests interleaved with long ones and lengths around
    the fixed cost (31, 32, 33, 64, 65) covers those boundaries."""
    runner, wl = mods
    rng = np.random.default_rng(79)
    lens = []
    for i in range(160):
        lens.append(1 if i % 3 else int(rng.choice([2, 31, 32, 33, 64, 65, 700, 5000, 20000])))
    S = 1 << 19
    rows = wl.rows_from_free_slots(rng.permutation(S), lens)
    w = wl.build_workload("decode-one-key-mix", "decode", torch.bfloat16, **wl.QWEN3_8B, page_size=1,
                          num_slots=S, max_running_req=len(lens), max_seq_len=20000, rows=rows, seq_lens=lens,
                          cached_lens=[L - 1 for L in lens], seed=79, q_std=1.0, device="cuda")
    say(f"[edges] one-key mix: {len(lens)} requests, {sum(lens)} keys, chunk {chunk}")
    res = runner.run_step(w, chunk=chunk)
    torch.cuda.synchronize()
    kp, vp, out_ref, lse_ref = oracle_mod.step(w)
    assert store_mismatch(w, res.k_pool, res.v_pool, kp, vp) == 0
    err = max_abs(res.out, out_ref)
    lse_err = max_abs(res.lse, lse_ref)
    say(f"[edges] one-key mix chunk {chunk}: max-abs {err:.3e} lse {lse_err:.2e}")
    assert err <= BF16_TOL and lse_err < 1e-3, (err, lse_err)
    # a one-key request returns its V row exactly (up to the bf16 rounding of V itself)
    one = [b for b, L in enumerate(lens) if L == 1][:20]
    for b in one:
        slot = int(w.page_table[int(w.table_idx[b]), 0])
        v = vp[slot].repeat_interleave(w.q_heads // w.kv_heads, dim=0)
        assert torch.equal(res.out[b].cpu().view(torch.int16), v.view(torch.int16)), b


@pytest.mark.parametrize("n_req,e_lo,e_hi", [(3, 1, 300), (2, 2048, 2100)])
def test_prefill_pool_beyond_4gib(mods, n_req, e_lo, e_hi):
    # a pool above 4 GiB (2^21 + 64 slots of 2 KB) runs the gathers' 64-bit
    # addressing; its first rows hold a small workload's pool, so the result
    # must equal, bit for bit, the same workload on the small pool (32-bit
    # offsets from the pool base), on both matrix-core layouts
    runner, wl = mods
    w = wl.ragged_prefill(device="cuda", n_req=n_req, e_lo=e_lo, e_hi=e_hi, c_lo=0, c_hi=300,
                          num_slots=1 << 13, seed=80 + e_lo)
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    runner.store_kv(w, kp, vp)
    big = (1 << 21) + 64
    kb = torch.zeros(big, w.kv_heads, w.head_dim, dtype=w.dtype, device="cuda")
    vb = torch.zeros_like(kb)
    kb[:kp.shape[0]] = kp
    vb[:vp.shape[0]] = vp
    assert kb.numel() * kb.element_size() > (1 << 32)
    say(f"[edge] prefill on a {kb.numel() * kb.element_size() / 2**30:.2f} GiB pool, T={w.num_tokens}")
    out_s, lse_s = runner.prefill_attn(w, kp, vp)
    out_b, lse_b = runner.prefill_attn(w, kb, vb)
    torch.cuda.synchronize()
    assert torch.equal(out_b.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_b, lse_s)
    del kb, vb
