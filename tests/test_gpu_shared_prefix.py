"""Cascade decode over shared radix prefixes (msgl_decode_attn_shared_prefix)
against the fp64 oracle's decode attention, and against the plain split-K
decode kernel on the same batch.

Bars as for decode: max-abs <= 2e-2 (bf16 outputs), lse within 1e-3, softmax
row sums from the returned lse within 1e-3 of 1.  The shared keys are read
once per group on matrix cores and merged with each request's own keys by the
log-sum-exp rule, so the result must equal ordinary decode attention."""

import pytest
import torch

from tests.gpu_util import BF16_TOL, ROWSUM_TOL, max_abs, rowsum_error, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import _lib, runner, workloads

    return _lib, runner, workloads


def _run(L, runner, sp, chunk=0):
    w = sp.w
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    runner.store_kv(w, kp, vp)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.bs, w.q_heads, dtype=torch.float32, device=w.q.device)
    ws = L.shared_prefix_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, chunk)
    L.msgl_decode_attn_shared_prefix(out, lse, w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens,
                                     sp.group_start, sp.prefix_lens, sp.max_group_size, sp.max_prefix_len,
                                     w.max_seq_len, ws, page_size=w.page_size, chunk=chunk)
    out_d, _ = runner.decode_attn(w, kp, vp, chunk=chunk)
    torch.cuda.synchronize()
    return out, lse, out_d


def _check(oracle_mod, mods, sp, chunk=0):
    L, runner, _ = mods
    w = sp.w
    say(f"[shared] {w.name} bs={w.bs} groups={sp.group_start.numel() - 1} max_prefix={sp.max_prefix_len} "
        f"H={w.q_heads} G={w.kv_heads} ps={w.page_size} ctx={int(w.seq_lens.sum())}")
    out, lse, out_d = _run(L, runner, sp, chunk)
    kp, vp, out_ref, lse_ref = oracle_mod.step(w)
    err = max_abs(out, out_ref)
    err_d = max_abs(out, out_d.double().cpu())
    lse_err = max_abs(lse, lse_ref)
    rs = rowsum_error(w, kp, vp, lse, range(w.bs))  # every request
    say(f"[shared] {w.name}: max-abs {err:.3e} (plain decode {err_d:.3e}), lse {lse_err:.2e}, rowsum {rs:.2e}")
    assert err <= BF16_TOL and err_d <= BF16_TOL, (err, err_d)
    assert lse_err < 1e-3, lse_err
    assert rs <= ROWSUM_TOL, rs


def test_four_groups_of_64_on_4096(oracle_mod, mods):
    _, _, wl = mods
    _check(oracle_mod, mods, wl.shared_prefix_decode(device="cuda"))


def test_sharp_queries(oracle_mod, mods):
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(32, 16), prefixes=(3000, 1500), singles=8,
                                 q_std=1.0, num_slots=1 << 18)
    _check(oracle_mod, mods, sp)


def test_page_size_16_uneven_groups(oracle_mod, mods):
    """Groups larger than one block's queries (40 > 32 at group size 4),
    small groups, prefixes of 1024 to 8192 tokens, page size 16."""
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(40, 64, 16, 8), prefixes=(4096, 2048, 1024, 8192),
                                 page_size=16, num_slots=1 << 20)
    _check(oracle_mod, mods, sp)


def test_ragged_prefixes_singletons_gqa2(oracle_mod, mods):
    """Prefixes that end inside a key tile (77, 1000, 130), one-request groups,
    requests in no group, Qwen3-0.6B heads (group size 2: 64 queries a block)."""
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(70, 1, 5, 1), prefixes=(1000, 77, 130, 1),
                                 singles=6, heads=wl.QWEN3_06B, num_slots=1 << 18, suffix_lo=1, suffix_hi=300)
    _check(oracle_mod, mods, sp)


def test_no_shared_prefix_is_plain_decode(oracle_mod, mods):
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(), prefixes=(), singles=24, num_slots=1 << 16)
    _check(oracle_mod, mods, sp)


@pytest.mark.parametrize("chunk", [64, 512])
def test_decode_split_sizes(oracle_mod, mods, chunk):
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(20, 12), prefixes=(2500, 640), singles=3,
                                 num_slots=1 << 17)
    _check(oracle_mod, mods, sp, chunk=chunk)


@pytest.mark.parametrize("H,G", [(8, 8), (64, 8)])
def test_group_sizes_one_and_eight(oracle_mod, mods, H, G):
    """GQA group sizes 1 and 8: 128 and 16 queries per prefix block."""
    _, _, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(40, 9), prefixes=(1500, 700), singles=2,
                                 heads=dict(H=H, G=G, d=128), num_slots=1 << 17, q_std=1.0)
    _check(oracle_mod, mods, sp)
