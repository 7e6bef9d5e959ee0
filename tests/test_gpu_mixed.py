"""The mixed multi-layer step at full size: 36 layers of Qwen3-8B attention
shapes, 192 lognormal decode requests plus 2 chunked prefills of 2048 tokens
on 8192-token prefixes, a pool of 60% of 288 GB at page_size 1, eager, per
layer store_kv then decode then prefill.

Attention parity against the oracle on layers 0, 17 and 35 (every decode row,
every 8th prefill row and each chunk's last, each as a one-query request at its own position);
store_kv on all 36 layers: every written row, plus sampled untouched history
rows regenerated from the seeded generator, plus sampled never-used slots.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import max_abs, oracle_rows, say

pytestmark = pytest.mark.gpu

CHECK_LAYERS = (0, 17, 35)


def test_mixed_step_36_layers(oracle_mod):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, total = torch.cuda.mem_get_info()
    if free < 190e9:
        pytest.skip(f"needs ~190 GB of free device memory, {free / 1e9:.0f} GB free")
    from paged_kv_attention_slots_amd import runner, workloads as wl

    say("[mixed] building 36 layers (pool 60% of 288 GB)")
    m = wl.mixed_step(device="cuda")
    say(f"[mixed] slots/layer={m.decode.num_slots} decode ctx={int(m.decode.seq_lens.sum())} "
        f"prefill lens={m.prefill.seq_lens.tolist()} T={m.num_tokens}")
    pre = {}
    for layer in CHECK_LAYERS:  # host copies of the state before the step
        pre[layer] = (m.k_pools[layer].cpu(), m.v_pools[layer].cpu())
    outs = {}
    for layer in range(m.layers):
        d, p = m.layer_views(layer)
        runner.store_kv(d, d.k_pool, d.v_pool)
        runner.store_kv(p, p.k_pool, p.v_pool)
        od, ld = runner.decode_attn(d, d.k_pool, d.v_pool)
        op, lp = runner.prefill_attn(p, p.k_pool, p.v_pool)
        if layer in CHECK_LAYERS:
            outs[layer] = (od, ld, op, lp)
    torch.cuda.synchronize()

    # store_kv, every layer
    rng = np.random.default_rng(0)
    loc = m.out_loc.long()
    dec_lens = m.decode.seq_lens.cpu()
    for layer in range(m.layers):
        kp, vp = m.k_pools[layer], m.v_pools[layer]
        assert torch.equal(kp[loc].view(torch.int16), m.k_new[layer].view(torch.int16)), layer
        assert torch.equal(vp[loc].view(torch.int16), m.v_new[layer].view(torch.int16)), layer
        b = int(rng.integers(0, m.decode.bs))
        pos = torch.from_numpy(rng.integers(0, int(dec_lens[b]) - 1, size=64))
        slots = m.decode.page_table[b, pos.cuda()].long()
        assert torch.equal(kp[slots].cpu().view(torch.int16),
                           wl.layer_history_values(m, layer, b, pos, "k").view(torch.int16)), layer
        assert torch.equal(vp[slots].cpu().view(torch.int16),
                           wl.layer_history_values(m, layer, b, pos, "v").view(torch.int16)), layer
    say("[mixed] store_kv checked on all layers")

    # never-used slots stay zero
    used = torch.zeros(m.decode.num_slots + 1, dtype=torch.bool)
    for w in (m.decode, m.prefill):
        for r in range(w.bs):
            used[w.page_table[int(w.table_idx[r]), :int(w.seq_lens[r])].cpu().long()] = True
    unused = torch.nonzero(~used[:-1]).flatten()
    pick = unused[torch.from_numpy(rng.choice(unused.numel(), size=4096, replace=False))].cuda()
    assert int(m.k_pools[5][pick].abs().sum()) == 0

    # attention parity on the checked layers
    for layer in CHECK_LAYERS:
        d, p = m.layer_views(layer)
        kp_h, vp_h = oracle_mod.store_kv(pre[layer][0], pre[layer][1], m.k_new[layer], m.v_new[layer],
                                         m.out_loc)
        od, ld, op, lp = outs[layer]
        ref, ref_lse = oracle_mod.attention(d.q, kp_h, vp_h, d.page_table, d.table_idx, d.seq_lens, d.cu_q)
        err = max_abs(od, ref)
        say(f"[mixed] layer {layer} decode: max-abs {err:.3e}")
        assert err <= 2e-2
        assert max_abs(ld, ref_lse) < 1e-3
        rows = np.concatenate([np.arange(0, p.num_tokens, 8), [p.num_tokens - 1, 2047, 2048]])
        rows = np.unique(rows)
        ref_p, ref_plse = oracle_rows(oracle_mod, p, kp_h, vp_h, rows)
        idx = torch.from_numpy(rows).cuda()
        err = max_abs(op[idx], ref_p)
        say(f"[mixed] layer {layer} prefill ({len(rows)} rows): max-abs {err:.3e}")
        assert err <= 2e-2
        assert max_abs(lp[idx], ref_plse) < 1e-3
        del kp_h, vp_h
