"""Parity of vocabulary indexing (msgl_vocab_embed) with the oracle: every
output row bit for bit, on whole tables and on tensor-parallel shards, with
ids outside the shard (zero rows), rows longer than one pass of the block,
ragged row lengths and more tokens than the grid holds blocks."""

import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_slots_amd import _lib, workloads

    return _lib, workloads


def _run(L, vb):
    out = torch.empty(vb.num_tokens, vb.hidden, dtype=vb.weight.dtype, device="cuda")
    out.fill_(float("nan"))  # a row the kernel skipped would show
    L.msgl_vocab_embed(out, vb.weight, vb.ids, vb.vocab_start)
    torch.cuda.synchronize()
    return out


def _check(oracle_mod, L, vb):
    say(f"[vocab] {vb.name} T={vb.num_tokens} rows={vb.weight.shape[0]} hidden={vb.hidden} "
        f"start={vb.vocab_start}")
    out = _run(L, vb)
    ref = oracle_mod.vocab_embed(vb.weight, vb.ids, vb.vocab_start)
    assert torch.equal(out.cpu().view(torch.uint8), ref.view(torch.uint8))
    return out


def test_vocab_qwen3_8b_table(oracle_mod, mods):
    L, wl = mods
    _check(oracle_mod, L, wl.vocab_batch(device="cuda"))


def test_vocab_decode_batch(oracle_mod, mods):
    L, wl = mods
    _check(oracle_mod, L, wl.vocab_batch(device="cuda", num_tokens=256, seed=7))


@pytest.mark.parametrize("shards", [2, 4])
def test_vocab_shards_sum_to_full_table(oracle_mod, mods, shards):
    L, wl = mods
    full = _check(oracle_mod, L, wl.vocab_batch(device="cuda", vocab=20000, hidden=1024))
    total = torch.zeros_like(full, dtype=torch.float32)
    for r in range(shards):
        part = _check(oracle_mod, L, wl.vocab_batch(device="cuda", vocab=20000, hidden=1024, shards=shards,
                                                     rank=r))
        total += part.float()
    assert torch.equal(total, full.float())


@pytest.mark.parametrize("hidden,dtype", [(64, torch.float32), (200, torch.float32), (12288, torch.bfloat16),
                                          (8, torch.bfloat16)])
def test_vocab_row_lengths(oracle_mod, mods, hidden, dtype):
    """16-byte rows, ragged vector counts (50), and rows of 1536 vectors (two
    passes of the block's threads)."""
    L, wl = mods
    _check(oracle_mod, L, wl.vocab_batch(device="cuda", vocab=3000, hidden=hidden, dtype=dtype,
                                         num_tokens=777, shards=3, rank=1))


def test_vocab_ids_outside_every_row(oracle_mod, mods):
    L, wl = mods
    vb = wl.vocab_batch(device="cuda", vocab=1000, hidden=64, num_tokens=64, shards=2, rank=1)
    vb.ids = torch.tensor([-2**31, -1, 0, 499, 500, 999, 1000, 2**31 - 1] * 8, dtype=torch.int32,
                          device="cuda")
    out = _check(oracle_mod, L, vb)
    assert torch.equal(out[2::8].float(), torch.zeros(8, 64, device="cuda"))


def test_vocab_more_tokens_than_blocks(oracle_mod, mods):
    L, wl = mods
    _check(oracle_mod, L, wl.vocab_batch(device="cuda", vocab=5000, hidden=64, num_tokens=70000))


def test_vocab_zero_tokens(mods):
    L, wl = mods
    vb = wl.vocab_batch(device="cuda", vocab=100, hidden=64, num_tokens=0)
    out = torch.empty(0, 64, dtype=vb.weight.dtype, device="cuda")
    L.msgl_vocab_embed(out, vb.weight, vb.ids, 0)
    torch.cuda.synchronize()
