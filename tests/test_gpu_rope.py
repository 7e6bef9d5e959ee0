"""Parity of the fused RoPE + KV write (msgl_rope_store_kv) with the fp64 oracle.

Bars.  V rows are copied bit for bit; pool rows the step does not write stay
bit-identical.  Rotated q and k values: the kernel takes the angles in double
precision, rounds cos and sin to float32 and rotates with float32 FMAs, so its
float32 value differs from the exact pair rotation by at most
4 * 2^-24 * (|x_i| + |x_{i+d/2}|) (two roundings of cos/sin, one product and
one FMA); the bar is twice that, delta = 2^-21 * (|x_i| + |x_{i+d/2}|).
fp32 outputs must lie within delta of the oracle; bf16 outputs, rounded once
to nearest even from that float32 value, within delta plus half a bf16 unit
in the last place of |oracle| + delta.  The rotated rows then feed attention,
which is held to the attention bars (2e-2 bf16).
"""

import math

import numpy as np
import pytest
import torch

from tests.gpu_util import max_abs, say, tol

pytestmark = pytest.mark.gpu

QWEN3_ROPE_BASE = 1e6


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


def rope_violation(x: torch.Tensor, ref: torch.Tensor, out: torch.Tensor) -> float:
    """max over elements of |out - ref| / bar (<= 1 passes); x is the input in
    its storage type, ref the oracle's fp64 rotation, out the kernel's."""
    x = x.cpu().to(torch.float64)
    half = x.shape[-1] // 2
    pair = x[..., :half].abs() + x[..., half:].abs()
    delta = 2.0 ** -21 * torch.cat([pair, pair], dim=-1)
    err = (out.cpu().to(torch.float64) - ref).abs()
    if out.dtype == torch.float32:
        bar = delta
    else:
        mag = (ref.abs() + delta).clamp_min(2.0 ** -126)
        _, e = torch.frexp(mag)  # mag = m * 2^e, m in [0.5, 1): one bf16 ulp is 2^(e - 8)
        bar = delta + 0.5 * torch.pow(2.0, (e - 8).to(torch.float64))
    if torch.isnan(err).any():
        return float("inf")
    return float((err / bar).max()) if err.numel() else 0.0


def _check(oracle_mod, runner, w, base, in_place=False):
    say(f"[rope] {w.name} T={w.num_tokens} H={w.q_heads} G={w.kv_heads} d={w.head_dim} "
        f"ps={w.page_size} base={base:g} in_place={in_place}")
    q_in = w.q.clone()
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    q_out = runner.rope_store_kv(w, kp, vp, base, q_out=w.q if in_place else None)
    torch.cuda.synchronize()
    pos = w.positions.cpu()
    q_ref = oracle_mod.rope(q_in.cpu(), pos, base)
    k_ref = oracle_mod.rope(w.k_new.cpu(), pos, base)
    loc = w.out_loc.long()
    vq = rope_violation(q_in, q_ref, q_out)
    vk = rope_violation(w.k_new, k_ref, kp[loc])
    say(f"[rope] {w.name}: q {vq:.3f} k {vk:.3f} of the bar")
    assert vq <= 1.0 and vk <= 1.0, (vq, vk)
    if w.dtype == torch.bfloat16:  # away from rounding ties the output is the rounded oracle value
        exact = (q_out.cpu() == q_ref.to(torch.float32).to(torch.bfloat16)).double().mean()
        assert exact >= 0.999, float(exact)
    # V rows bit for bit; every other pool row untouched
    assert torch.equal(vp[loc].view(torch.uint8), w.v_new.view(torch.uint8))
    kp[loc] = w.k_pool[loc]
    vp[loc] = w.v_pool[loc]
    assert torch.equal(kp.view(torch.uint8), w.k_pool.view(torch.uint8))
    assert torch.equal(vp.view(torch.uint8), w.v_pool.view(torch.uint8))
    return q_out


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_rope_tiny_fp32(oracle_mod, runner, wl, mode):
    _check(oracle_mod, runner, wl.tiny(mode, device="cuda"), 1e4)


def test_rope_qwen3_06b_decode(oracle_mod, runner, wl):
    _check(oracle_mod, runner, wl.qwen3_06b_decode(device="cuda"), QWEN3_ROPE_BASE)


def test_rope_ragged_prefill(oracle_mod, runner, wl):
    _check(oracle_mod, runner, wl.ragged_prefill(device="cuda"), QWEN3_ROPE_BASE)


def test_rope_qwen3_8b_decode_ps16_in_place(oracle_mod, runner, wl):
    _check(oracle_mod, runner, wl.qwen3_8b_decode(page_size=16, device="cuda"), QWEN3_ROPE_BASE,
           in_place=True)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 128), (torch.bfloat16, 128), (torch.bfloat16, 64)])
def test_rope_far_positions(oracle_mod, runner, wl, dtype, d):
    """Positions up to 2^24: angles of millions of radians, reduced in double."""
    w = wl.tiny("prefill", device="cuda", dtype=dtype, lens=(300, 200), d=d, H=8, G=2,
                num_slots=1024)
    g = torch.Generator().manual_seed(5)
    w.positions = torch.randint(0, 1 << 24, (w.num_tokens,), generator=g, dtype=torch.int32).cuda()
    _check(oracle_mod, runner, w, 1e4)


def test_rope_invalid_slot_writes_no_row(oracle_mod, runner, wl):
    """A token whose out_loc is outside the pool still has its q turned and
    writes nothing (the kernel's own bounds check)."""
    w = wl.tiny("prefill", device="cuda")
    loc = w.out_loc.clone()
    loc[3] = -1
    loc[7] = w.k_pool.shape[0]
    w.out_loc = loc
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    q_out = runner.rope_store_kv(w, kp, vp, 1e4)
    torch.cuda.synchronize()
    q_ref = oracle_mod.rope(w.q.cpu(), w.positions.cpu(), 1e4)
    assert rope_violation(w.q, q_ref, q_out) <= 1.0
    ok = torch.ones(w.num_tokens, dtype=torch.bool)
    ok[3] = ok[7] = False
    good = loc[ok.cuda()].long()
    assert torch.equal(vp[good], w.v_new[ok.cuda()])
    kp[good] = w.k_pool[good]
    vp[good] = w.v_pool[good]
    assert torch.equal(kp, w.k_pool) and torch.equal(vp, w.v_pool)


def test_rope_zero_tokens(runner, wl):
    w = wl.tiny("decode", device="cuda")
    from paged_kv_attention_slots_amd import _lib

    e = torch.empty(0, dtype=torch.int32, device="cuda")
    q = torch.empty(0, w.q_heads, w.head_dim, device="cuda")
    kv = torch.empty(0, w.kv_heads, w.head_dim, device="cuda")
    kp = w.k_pool.clone()
    _lib.msgl_rope_store_kv(q, q, kp, w.v_pool, kv, kv, e, e, 1e4)
    torch.cuda.synchronize()
    assert torch.equal(kp, w.k_pool)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_rope_then_attention(oracle_mod, runner, wl, mode):
    """The layer's RoPE -> KV write -> attention, against the oracle's same
    chain (rotations in fp64, rounded once to the storage type)."""
    if mode == "decode":
        w = wl.qwen3_06b_decode(device="cuda", bs=16, q_std=1.0)
    else:
        w = wl.ragged_prefill(device="cuda", n_req=3, e_lo=100, e_hi=300, c_lo=0, c_hi=200,
                              q_std=1.0)
    base = QWEN3_ROPE_BASE
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    q_rot = runner.rope_store_kv(w, kp, vp, base)
    w_gpu = type(w)(**{**w.__dict__, "q": q_rot})
    if mode == "decode":
        out, _ = runner.decode_attn(w_gpu, kp, vp)
    else:
        out, _ = runner.prefill_attn(w_gpu, kp, vp)
    torch.cuda.synchronize()
    pos = w.positions.cpu()
    q_ref = oracle_mod.rope(w.q.cpu(), pos, base).to(torch.float32).to(w.dtype)
    k_ref = oracle_mod.rope(w.k_new.cpu(), pos, base).to(torch.float32).to(w.dtype)
    kp_ref, vp_ref = oracle_mod.store_kv(w.k_pool, w.v_pool, k_ref, w.v_new, w.out_loc)
    out_ref, _ = oracle_mod.attention(q_ref, kp_ref, vp_ref, w.page_table, w.table_idx, w.seq_lens,
                                      w.cu_q)
    err = max_abs(out, out_ref)
    say(f"[rope] {w.name} rope->store->{mode}: max-abs {err:.3e}")
    assert err <= tol(w), err
