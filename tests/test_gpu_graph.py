"""The captured decode step (store_kv + decode attention as one HIP graph).

Mirrors the padded replay the Stage 4 milestone prints (3 requests padded to
a recorded batch of 4, replayed for 5 rounds, same output as without the
graph) and its fixed-buffer discipline: a value written anywhere but the
recorded buffer is not seen by the replay, one written into it is.
"""

import pytest
import torch

from tests.gpu_util import max_abs, say, store_mismatch

pytestmark = pytest.mark.gpu

ROUNDS = 5


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import _lib, runner, workloads

    return _lib, runner, workloads


def _round_inputs(wl, w, r, real, rounds):
    """Decode round r of the first `real` requests: every request is r tokens
    longer than at round 0 (the last round ends at the workload's lengths); its
    new token sits at position seq_len - 1."""
    seq = (w.seq_lens[:real] - rounds + 1 + r).clone()
    rows = w.table_idx[:real]
    loc = w.page_table[rows.long(), (seq - 1).long()].to(torch.int32)
    tok = torch.arange(real, dtype=torch.int64) + 1000 * (r + 1)
    G, H, d = w.kv_heads, w.q_heads, w.head_dim
    k_new = wl.gen_rows(w.seed, 11, tok, G * d, 1.0, w.dtype, w.q.device).view(real, G, d)
    v_new = wl.gen_rows(w.seed, 12, tok, G * d, 1.0, w.dtype, w.q.device).view(real, G, d)
    q = wl.gen_rows(w.seed, 13, tok, H * d, 1.0 / 8.0, w.dtype, w.q.device).view(real, H, d)
    return seq, loc, k_new, v_new, q


def _check_padded_replay(oracle_mod, mods, base, page_size, real, padded, rounds):
    """Record the step at `padded` rows, run `rounds` decode rounds of the
    first `real` requests through it and through the eager calls; the real
    rows must be bit-identical to eager and within 2e-2 of the oracle in every
    round, and every pool slot but the dummy page's bit-exact at the end."""
    _lib, runner, wl = mods
    dev = torch.device("cuda")
    say(f"[graph] ps={page_size} real={real} padded={padded} rounds={rounds} "
        f"ctx={int(base.seq_lens[:real].sum())}")
    # fixed buffers at the padded size, dummy rows prefilled
    pad = wl.pad_decode(wl.subset_decode(base, real), padded)
    buf = {k: getattr(pad, k).clone() for k in ("q", "k_new", "v_new", "out_loc", "table_idx", "seq_lens")}
    out = torch.zeros_like(buf["q"])
    lse = torch.zeros(padded, base.q_heads, dtype=torch.float32, device=dev)
    ws = _lib.decode_workspace(padded, base.q_heads, base.head_dim, base.max_seq_len, device=dev)
    kp = base.k_pool.clone()
    vp = base.v_pool.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = _lib.msgl_decode_graph_create(kp, vp, buf["k_new"], buf["v_new"], buf["out_loc"], out, lse, buf["q"],
                                      base.page_table, buf["table_idx"], buf["seq_lens"], base.max_seq_len,
                                      ws, page_size=page_size, stream=stream)
    # eager twin with its own pools and workspace
    kp_e = base.k_pool.clone()
    vp_e = base.v_pool.clone()
    kp_h = base.k_pool.cpu()
    vp_h = base.v_pool.cpu()
    for r in range(rounds):
        seq, loc, k_new, v_new, q = _round_inputs(wl, base, r, real, rounds)
        # copy this round's values into the recorded buffers (real rows only)
        buf["seq_lens"][:real].copy_(seq)
        buf["out_loc"][:real].copy_(loc)
        buf["k_new"][:real].copy_(k_new)
        buf["v_new"][:real].copy_(v_new)
        buf["q"][:real].copy_(q)
        torch.cuda.synchronize()  # the copies ran on the default stream
        g.launch(stream)
        stream.synchronize()
        # eager twin: the same padded batch through the eager entry points
        step = wl.pad_decode(wl.subset_decode(base, real), padded)
        for k in ("q", "k_new", "v_new", "out_loc", "table_idx", "seq_lens"):
            setattr(step, k, buf[k].clone())
        step.cached_lens = step.seq_lens - 1
        runner.store_kv(step, kp_e, vp_e)
        out_e, lse_e = runner.decode_attn(step, kp_e, vp_e)
        torch.cuda.synchronize()
        assert torch.equal(out[:real].view(torch.int16), out_e[:real].view(torch.int16)), f"round {r}"
        assert torch.equal(lse[:real], lse_e[:real])
        # oracle on host copies of the same inputs
        kp_h, vp_h = oracle_mod.store_kv(kp_h, vp_h, k_new, v_new, loc)
        ref, ref_lse = oracle_mod.attention(q, kp_h, vp_h, base.page_table, base.table_idx[:real], seq,
                                            torch.arange(real + 1, dtype=torch.int32))
        err = max_abs(out[:real], ref)
        say(f"[graph] round {r}: max-abs vs oracle {err:.3e}")
        assert err <= 2e-2
        assert max_abs(lse[:real], ref_lse) < 1e-3
    assert store_mismatch(base, kp, vp, kp_h, vp_h) == 0
    g.destroy()


@pytest.mark.parametrize("page_size,real,padded", [(1, 3, 4), (16, 3, 4), (16, 100, 128)])
def test_graph_padded_replay_matches_eager_and_oracle(oracle_mod, mods, page_size, real, padded):
    wl = mods[2]
    base = wl.qwen3_8b_decode(page_size=page_size, device=torch.device("cuda"), bs=padded, median=700.0,
                              hi=8192, num_slots=1 << 20)
    _check_padded_replay(oracle_mod, mods, base, page_size, real, padded, ROUNDS)


# The Qwen3-8B decode batch at full size (256 requests, lognormal lengths up to
# 32768, 2^21 slots), built once per page size and shared by the tests below.
_CONFIG4 = {}


def _config4(wl, page_size):
    if page_size not in _CONFIG4:
        _CONFIG4.clear()  # one page size resident at a time
        torch.cuda.empty_cache()
        _CONFIG4[page_size] = wl.qwen3_8b_decode(page_size=page_size, device=torch.device("cuda"))
    return _CONFIG4[page_size]


@pytest.mark.parametrize("page_size", [1, 16])
def test_graph_full_batch_config4(oracle_mod, mods, page_size):
    # the captured step at the recorded size 256 with all 256 lognormal
    # requests: the shape the throughput figure is taken on
    base = _config4(mods[2], page_size)
    _check_padded_replay(oracle_mod, mods, base, page_size, 256, 256, 3)


@pytest.mark.parametrize("page_size", [1, 16])
@pytest.mark.parametrize("real,padded", [(1, 1), (2, 2), (7, 8), (16, 16), (30, 32), (64, 64), (200, 256)])
def test_graph_recorded_sizes_config4(oracle_mod, mods, page_size, real, padded):
    # every other recorded batch size on the same lognormal batch (its first
    # `real` requests), exactly full or padded with dummy rows
    base = _config4(mods[2], page_size)
    _check_padded_replay(oracle_mod, mods, base, page_size, real, padded, 2)


def test_graph_reads_only_recorded_buffers(mods):
    _lib, runner, wl = mods
    dev = torch.device("cuda")
    w = wl.pad_decode(wl.qwen3_8b_decode(page_size=1, device=dev, bs=3, median=500.0, hi=4096,
                                         num_slots=1 << 16), 4)
    out = torch.zeros_like(w.q)
    ws = _lib.decode_workspace(4, w.q_heads, w.head_dim, w.max_seq_len, device=dev)
    kp, vp = w.k_pool.clone(), w.v_pool.clone()
    q_buf = w.q.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = _lib.msgl_decode_graph_create(kp, vp, w.k_new, w.v_new, w.out_loc, out, None, q_buf, w.page_table,
                                      w.table_idx, w.seq_lens, w.max_seq_len, ws, stream=stream)
    g.launch(stream)
    stream.synchronize()
    first = out.clone()
    # a new q written to a different tensor: the replay still reads the recorded one
    q_other = torch.flip(w.q, dims=[0]).contiguous()
    g.launch(stream)
    stream.synchronize()
    assert torch.equal(out.view(torch.int16), first.view(torch.int16))
    # written into the recorded buffer: the replay follows
    q_buf.copy_(q_other)
    torch.cuda.synchronize()
    g.launch(stream)
    stream.synchronize()
    assert not torch.equal(out[:3].view(torch.int16), first[:3].view(torch.int16))
    w2 = w.to(dev)
    w2.q = q_other
    ref, _ = runner.decode_attn(w2, kp, vp)
    torch.cuda.synchronize()
    assert torch.equal(out[:3].view(torch.int16), ref[:3].view(torch.int16))
    g.destroy()
