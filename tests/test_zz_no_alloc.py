"""The allocation-free decode call (msgl_decode_attn_noalloc), whose workspace
is the library's fixed device scratch, against msgl_decode_attn with a caller
workspace: the same kernels, so the outputs must agree bit for bit.  Two calls
in a row share the scratch, the second on a smaller batch (the first call's
contents must not leak into it).  Through the C ABI (the ctypes binding)."""

import pytest
import torch

from tests.gpu_util import max_abs, say


def _both(runner, _lib, w, kp, vp):
    out_w = torch.full_like(w.q, float("nan"))
    lse_w = torch.full((w.bs, w.q_heads), float("nan"), dtype=torch.float32, device=w.q.device)
    ws = _lib.decode_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len, device=w.q.device)
    _lib.msgl_decode_attn(out_w, lse_w, w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens, w.max_seq_len, ws,
                          page_size=w.page_size, sm_scale=w.sm_scale)
    out_n = torch.full_like(w.q, float("nan"))
    lse_n = torch.full((w.bs, w.q_heads), float("nan"), dtype=torch.float32, device=w.q.device)
    _lib.msgl_decode_attn_noalloc(out_n, lse_n, w.q, kp, vp, w.page_table, w.table_idx, w.seq_lens,
                                  w.max_seq_len, page_size=w.page_size, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    return out_w, lse_w, out_n, lse_n


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_call(oracle_mod):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import _lib, runner, workloads as wl

    dev = torch.device("cuda")
    cases = [
        # the Qwen3-8B decode batch at full size, page size 16 (72 MB of workspace)
        wl.qwen3_8b_decode(page_size=16, device=dev),
        # then a smaller one: 24 Qwen3-0.6B-shaped requests
        wl.qwen3_06b_decode(device=dev, bs=24, lo=100, hi=1500, num_slots=1 << 16),
    ]
    for w in cases:
        need = _lib.msgl_decode_workspace_bytes(w.bs, w.q_heads, w.head_dim, w.max_seq_len)
        say(f"[noalloc] {w.name} bs={w.bs} H={w.q_heads} ps={w.page_size}: workspace {need} of "
            f"{_lib.msgl_noalloc_scratch_bytes()} scratch bytes")
        assert need <= _lib.msgl_noalloc_scratch_bytes()
        kp, vp = w.k_pool.clone(), w.v_pool.clone()
        runner.store_kv(w, kp, vp)
        out_w, lse_w, out_n, lse_n = _both(runner, _lib, w, kp, vp)
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16)), w.name
        assert torch.equal(lse_n, lse_w), w.name
        if w.bs <= 64:  # and the oracle, where it is quick
            kp_h, vp_h = oracle_mod.store_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.out_loc)
            ref, _ = oracle_mod.attention(w.q, kp_h, vp_h, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
            err = max_abs(out_n, ref)
            say(f"[noalloc] {w.name}: max-abs vs oracle {err:.3e}")
            assert err <= 2e-2
        del kp, vp


def test_noalloc_rejects_batches_beyond_the_scratch():
    # argument checks only: nothing is launched, no GPU is needed
    from paged_kv_attention_slots_amd import _lib

    lib = _lib.lib
    fake = 0x10000
    args = lambda bs, H: (fake, None, fake, fake, fake, 1 << 20, fake, 4096, fake, fake, bs, H, 8, 128, 1, 4096, 0,
                          0.088, _lib.MSGL_BF16, None)
    st = lib.msgl_decode_attn_noalloc(*args(945, 32))
    assert st == _lib.MSGL_WORKSPACE_TOO_SMALL and "scratch" in _lib.msgl_last_error()
    assert lib.msgl_decode_attn_noalloc(*args(10, 64)) == _lib.MSGL_WORKSPACE_TOO_SMALL
    assert lib.msgl_decode_workspace_bytes(944, 32, 128, 4096, 0) <= _lib.msgl_noalloc_scratch_bytes()
    # the other checks of msgl_decode_attn still apply
    assert lib.msgl_decode_attn_noalloc(*args(-1, 32)) == _lib.MSGL_INVALID_ARG
    # an empty batch is a no-op
    assert lib.msgl_decode_attn_noalloc(*args(0, 32)) == _lib.MSGL_OK
