"""Planned prefill (host plan / run split): the launch reads each block's work
item from the host-made plan instead of enumerating the batch on the device.
Every block computes what it computes unplanned, so the outputs equal
msgl_prefill_attn's bit for bit; against the fp64 oracle they meet the bf16
bar.  A batch beyond the 1024 requests of the device enumeration runs on the
matrix cores only when planned."""

import numpy as np
import pytest
import torch

from tests.gpu_util import max_abs, oracle_rows, sample_rows, say, store_mismatch, tol

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


def _stored(runner, w):
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    runner.store_kv(w, kp, vp)
    return kp, vp


def _same_as_unplanned(runner, w):
    kp, vp = _stored(runner, w)
    out0, lse0 = runner.prefill_attn(w, kp, vp)
    plan = runner.prefill_plan(w)
    say(f"[plan] {w.name} bs={w.bs} T={w.num_tokens} H={w.q_heads} G={w.kv_heads} ps={w.page_size}: "
        f"layout {int(plan[0][1])}, {int(plan[0][3])} entries")
    out1, lse1 = runner.prefill_attn_planned(w, kp, vp, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0, lse1)
    return kp, vp, out1, lse1


@pytest.mark.parametrize("case", ["config3", "qwen3_8b_heads", "page16", "gqa1", "gqa8"])
def test_planned_equals_unplanned(runner, wl, case):
    if case == "config3":
        w = wl.ragged_prefill(device="cuda")
    elif case == "qwen3_8b_heads":
        w = wl.ragged_prefill(device="cuda", seed=61, heads=dict(H=32, G=8, d=128))
    elif case == "page16":
        w = wl.ragged_prefill(device="cuda", n_req=5, e_lo=1, e_hi=700, c_lo=0, c_hi=500, num_slots=1 << 14,
                              seed=62, page_size=16)
    elif case == "gqa1":
        w = wl.ragged_prefill(device="cuda", n_req=4, e_lo=1, e_hi=300, c_lo=0, c_hi=200, num_slots=1 << 12,
                              seed=63, heads=dict(H=8, G=8, d=128))
    else:
        w = wl.ragged_prefill(device="cuda", n_req=4, e_lo=1, e_hi=300, c_lo=0, c_hi=200, num_slots=1 << 12,
                              seed=64, heads=dict(H=64, G=8, d=128))
    _same_as_unplanned(runner, w)


def test_planned_long_layout(runner, wl):
    # two 2048-token chunks on 8192-token cached prefixes: the single-block layout
    w = wl.ragged_prefill(device="cuda", n_req=2, e_lo=2048, e_hi=2048, c_lo=8192, c_hi=8192,
                          num_slots=1 << 15, seed=65, heads=dict(H=32, G=8, d=128))
    kp, vp, out, lse = _same_as_unplanned(runner, w)


def test_planned_against_oracle(oracle_mod, runner, wl):
    w = wl.ragged_prefill(device="cuda", n_req=4, e_lo=1, e_hi=300, c_lo=0, c_hi=200, num_slots=1 << 12, seed=66)
    kp, vp = _stored(runner, w)
    out, lse = runner.prefill_attn_planned(w, kp, vp)
    torch.cuda.synchronize()
    kp_ref, vp_ref, out_ref, lse_ref = oracle_mod.step(w)
    assert store_mismatch(w, kp, vp, kp_ref, vp_ref) == 0
    err = max_abs(out, out_ref)
    say(f"[plan] {w.name} against the oracle: max-abs {err:.3e}")
    assert err <= tol(w), err
    assert max_abs(lse, lse_ref) < 1e-3


def test_planned_beyond_device_enumeration(oracle_mod, runner, wl):
    # 1100 requests: unplanned, the vector-ALU kernel serves them; planned, the matrix-core kernel
    w = wl.ragged_prefill(device="cuda", n_req=1100, e_lo=1, e_hi=6, c_lo=0, c_hi=60, num_slots=1 << 17, seed=67)
    kp, vp = _stored(runner, w)
    out, lse = runner.prefill_attn_planned(w, kp, vp)
    torch.cuda.synchronize()
    kp_ref, vp_ref = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
    rows = sample_rows(w, 256)
    out_ref, lse_ref = oracle_rows(oracle_mod, w, kp_ref, vp_ref, rows)
    idx = torch.from_numpy(rows).cuda()
    err = max_abs(out[idx], out_ref)
    say(f"[plan] {w.bs} requests, sampled {len(rows)} rows: max-abs {err:.3e}")
    assert err <= tol(w), err
    assert max_abs(lse[idx], lse_ref) < 1e-3


def test_planned_single_new_tokens_and_full_row(runner, wl):
    # one-token extends, tile-edge lengths, and a request whose keys fill its whole 32768-entry row
    cached = [0, 5, 32700, 0, 63, 64]
    ext = [1, 1, 68, 130, 1, 65]
    lens = [c + e for c, e in zip(cached, ext)]
    rng = np.random.default_rng(79)
    rows = wl.rows_from_free_slots(rng.permutation(1 << 16), lens, new_after_history=False)
    w = wl.build_workload("prefill-edges", "prefill", torch.bfloat16, **wl.QWEN3_06B, page_size=1,
                          num_slots=1 << 16, max_running_req=len(lens), max_seq_len=32768, rows=rows,
                          seq_lens=lens, cached_lens=cached, seed=79, q_std=1.0, device="cuda")
    assert max(lens) == w.row_stride
    _same_as_unplanned(runner, w)


def test_planned_long_layout_page16(runner, wl):
    # the single-block layout over shuffled 16-token pages
    w = wl.ragged_prefill(device="cuda", n_req=2, e_lo=2100, e_hi=2600, c_lo=300, c_hi=3000, num_slots=1 << 14,
                          seed=68, page_size=16, heads=dict(H=16, G=8, d=128))
    plan = runner.prefill_plan(w)
    assert int(plan[0][1]) == 1
    _same_as_unplanned(runner, w)
