"""The layer's decode path captured as one HIP graph through the C ABI: fused
RoPE + KV write, then cascade attention over shared prefixes.  Every call
only enqueues kernels (no allocation, no host synchronisation), so torch's
stream capture records them as they are.  The graph is replayed for several
rounds, with new inputs written into the recorded buffers and eager work in
between; each replay must equal the same calls run eagerly (bit for bit) and
the oracle's RoPE -> store -> attention chain (2e-2)."""

import pytest
import torch

from tests.gpu_util import BF16_TOL, max_abs, say

pytestmark = pytest.mark.gpu

ROUNDS = 3
ROPE_BASE = 1e6


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import _lib, workloads

    return _lib, workloads


def test_rope_store_cascade_graph_replays(oracle_mod, mods):
    L, wl = mods
    sp = wl.shared_prefix_decode(device="cuda", group_sizes=(24, 8), prefixes=(2048, 512), singles=4,
                                 num_slots=1 << 17, q_std=1.0)
    w = sp.w
    say(f"[graph-layer] bs={w.bs} groups=2 ctx={int(w.seq_lens.sum())}")
    # recorded (fixed) input buffers
    q_in, k_in, v_in = w.q.clone(), w.k_new.clone(), w.v_new.clone()

    def state():
        return {"kp": w.k_pool.clone(), "vp": w.v_pool.clone(), "q_rot": torch.empty_like(q_in),
                "out": torch.empty_like(q_in),
                "lse": torch.empty(w.bs, w.q_heads, dtype=torch.float32, device="cuda"),
                "ws": L.shared_prefix_workspace(w.bs, w.q_heads, w.head_dim, w.max_seq_len)}

    def layer(s):
        L.msgl_rope_store_kv(s["q_rot"], q_in, s["kp"], s["vp"], k_in, v_in, w.positions, w.out_loc, ROPE_BASE)
        L.msgl_decode_attn_shared_prefix(s["out"], s["lse"], s["q_rot"], s["kp"], s["vp"], w.page_table,
                                         w.table_idx, w.seq_lens, sp.group_start, sp.prefix_lens,
                                         sp.max_group_size, sp.max_prefix_len, w.max_seq_len, s["ws"])

    g_state, e_state = state(), state()
    layer(g_state)  # eager first call: the library resolves its cached device queries outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer(g_state)
    torch.cuda.synchronize()

    kp_h, vp_h = w.k_pool.cpu(), w.v_pool.cpu()
    for r in range(ROUNDS):
        tok = torch.arange(w.bs, dtype=torch.int64) + 5000 * (r + 1)
        G, H, d = w.kv_heads, w.q_heads, w.head_dim
        q_in.copy_(wl.gen_rows(w.seed, 21, tok, H * d, 1.0, w.dtype, "cuda").view(w.bs, H, d))
        k_in.copy_(wl.gen_rows(w.seed, 22, tok, G * d, 1.0, w.dtype, "cuda").view(w.bs, G, d))
        v_in.copy_(wl.gen_rows(w.seed, 23, tok, G * d, 1.0, w.dtype, "cuda").view(w.bs, G, d))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        layer(e_state)
        torch.cuda.synchronize()
        for k in ("q_rot", "out", "kp", "vp"):
            assert torch.equal(g_state[k].view(torch.uint8), e_state[k].view(torch.uint8)), (r, k)
        assert torch.equal(g_state["lse"], e_state["lse"]), r
        # the oracle's chain: rotations in fp64 rounded once to bf16, store, attention
        pos = w.positions.cpu()
        q_ref = oracle_mod.rope(q_in, pos, ROPE_BASE).to(torch.float32).to(w.dtype)
        k_ref = oracle_mod.rope(k_in, pos, ROPE_BASE).to(torch.float32).to(w.dtype)
        kp_h, vp_h = oracle_mod.store_kv(kp_h, vp_h, k_ref, v_in, w.out_loc)
        ref, _ = oracle_mod.attention(q_ref, kp_h, vp_h, w.page_table, w.table_idx, w.seq_lens, w.cu_q)
        err = max_abs(g_state["out"], ref)
        say(f"[graph-layer] round {r}: replay == eager, max-abs vs oracle {err:.3e}")
        assert err <= BF16_TOL, (r, err)
