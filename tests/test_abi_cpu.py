"""The C ABI library loads and exports every declared symbol, and its host-side
logic (argument checks, status codes, the batch validator) works without a GPU.
No call here reaches a kernel launch: every compute call below fails its
argument checks first."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msgl.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msgl_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from paged_kv_attention_slots_amd import _lib

    return _lib


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    assert set(names) == set(L.EXPORTS)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_error_text(L):
    assert L.msgl_version() >= 100
    assert isinstance(L.msgl_last_error(), str)


FAKE = 0x10000  # never dereferenced: every call below is rejected before launch


def test_store_kv_argument_checks(L):
    lib = L.lib
    st = lib.msgl_store_kv(FAKE, FAKE, 100, 8, 96, 1, FAKE, FAKE, FAKE, 4, None)
    assert st == L.MSGL_UNSUPPORTED and "head_dim" in L.msgl_last_error()
    st = lib.msgl_store_kv(FAKE, FAKE, 100, 8, 128, 7, FAKE, FAKE, FAKE, 4, None)
    assert st == L.MSGL_UNSUPPORTED
    st = lib.msgl_store_kv(None, FAKE, 100, 8, 128, 1, FAKE, FAKE, FAKE, 4, None)
    assert st == L.MSGL_INVALID_ARG
    st = lib.msgl_store_kv(FAKE, FAKE, 100, 8, 128, 1, FAKE, FAKE, FAKE, -1, None)
    assert st == L.MSGL_INVALID_ARG
    st = lib.msgl_store_kv(FAKE, FAKE, 0, 8, 128, 1, FAKE, FAKE, FAKE, 1, None)
    assert st == L.MSGL_INVALID_ARG
    # zero tokens is a no-op that needs no pointers and no GPU
    assert lib.msgl_store_kv(None, None, 100, 8, 128, 1, None, None, None, 0, None) == L.MSGL_OK


def test_vocab_embed_argument_checks(L):
    lib = L.lib

    def call(out=FAKE, w=FAKE, start=0, rows=1000, hid=4096, dt=1, ids=FAKE, T=4):
        return lib.msgl_vocab_embed(out, w, start, rows, hid, dt, ids, T, None)

    assert call(hid=4) == L.MSGL_UNSUPPORTED and "16" in L.msgl_last_error()  # 8-byte bf16 rows
    assert call(dt=3) == L.MSGL_UNSUPPORTED
    assert call(hid=0) == L.MSGL_INVALID_ARG
    assert call(rows=0) == L.MSGL_INVALID_ARG
    assert call(start=-1) == L.MSGL_INVALID_ARG
    assert call(T=-1) == L.MSGL_INVALID_ARG
    assert call(ids=None) == L.MSGL_INVALID_ARG and "NULL" in L.msgl_last_error()
    assert call(out=None) == L.MSGL_INVALID_ARG
    assert call(None, None, ids=None, T=0) == L.MSGL_OK


def test_rope_store_kv_argument_checks(L):
    lib = L.lib

    def call(q_out=FAKE, q=FAKE, k=FAKE, v=FAKE, S=100, H=32, G=8, d=128, dt=1, kn=FAKE, vn=FAKE,
             pos=FAKE, loc=FAKE, T=4, base=1e6):
        return lib.msgl_rope_store_kv(q_out, q, k, v, S, H, G, d, dt, kn, vn, pos, loc, T, base, None)

    assert call(d=96) == L.MSGL_UNSUPPORTED and "head_dim" in L.msgl_last_error()
    assert call(dt=5) == L.MSGL_UNSUPPORTED
    assert call(H=0) == L.MSGL_INVALID_ARG and "q_heads" in L.msgl_last_error()
    assert call(base=0.0) == L.MSGL_INVALID_ARG and "rope_base" in L.msgl_last_error()
    assert call(base=-1e4) == L.MSGL_INVALID_ARG
    assert call(base=float("inf")) == L.MSGL_INVALID_ARG
    assert call(base=float("nan")) == L.MSGL_INVALID_ARG
    assert call(pos=None) == L.MSGL_INVALID_ARG and "NULL" in L.msgl_last_error()
    assert call(q_out=None) == L.MSGL_INVALID_ARG
    assert call(k=None) == L.MSGL_INVALID_ARG
    assert call(T=-1) == L.MSGL_INVALID_ARG
    assert call(S=0) == L.MSGL_INVALID_ARG
    # zero tokens is a no-op that needs no pointers and no GPU
    assert call(None, None, None, None, kn=None, vn=None, pos=None, loc=None, T=0) == L.MSGL_OK


def _decode(L, **over):
    a = dict(out=FAKE, lse=None, q=FAKE, k=FAKE, v=FAKE, S=1000, pt=FAKE, W=4096, tix=FAKE, sl=FAKE,
             bs=4, H=32, G=8, d=128, ps=1, msl=4096, chunk=0, scale=0.088, dt=1, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return L.lib.msgl_decode_attn(a["out"], a["lse"], a["q"], a["k"], a["v"], a["S"], a["pt"], a["W"],
                                  a["tix"], a["sl"], a["bs"], a["H"], a["G"], a["d"], a["ps"], a["msl"],
                                  a["chunk"], a["scale"], a["dt"], a["ws"], a["wsb"], None)


def test_decode_argument_checks(L):
    assert _decode(L, H=12) == L.MSGL_INVALID_ARG  # not a multiple of kv_heads
    assert _decode(L, H=30) == L.MSGL_INVALID_ARG
    assert _decode(L, H=8 * 16) == L.MSGL_UNSUPPORTED  # group 16
    assert _decode(L, d=80) == L.MSGL_UNSUPPORTED
    assert _decode(L, q=None) == L.MSGL_INVALID_ARG
    assert _decode(L, msl=5000) == L.MSGL_INVALID_ARG  # beyond row_stride
    assert _decode(L, chunk=100) == L.MSGL_INVALID_ARG
    assert _decode(L, ps=0) == L.MSGL_INVALID_ARG
    need = L.msgl_decode_workspace_bytes(4, 32, 128, 4096)
    assert need > 0
    assert _decode(L, wsb=need - 1) == L.MSGL_WORKSPACE_TOO_SMALL
    assert "workspace" in L.msgl_last_error()
    assert _decode(L, bs=-1) == L.MSGL_INVALID_ARG
    assert _decode(L, bs=100000) == L.MSGL_UNSUPPORTED


def test_decode_workspace_size_formula(L):
    # control block + length prefix + (m, l, o[d]) float32 per (piece, q head),
    # with at most batch + 4096 pieces
    bs, H, d, msl = 256, 32, 128, 32768
    prefix = ((bs + 1) * 4 + 255) // 256 * 256
    assert L.msgl_decode_workspace_bytes(bs, H, d, msl, 256) == 256 + prefix + (bs + 4096) * H * (d + 2) * 4
    assert L.msgl_decode_workspace_bytes(bs, H, d, msl, 0) == L.msgl_decode_workspace_bytes(bs, H, d, msl, 256)


def _prefill(L, **over):
    a = dict(out=FAKE, lse=None, q=FAKE, k=FAKE, v=FAKE, S=1000, pt=FAKE, W=4096, tix=FAKE, sl=FAKE,
             cl=FAKE, cu=FAKE, bs=2, T=10, me=8, H=16, G=8, d=128, ps=1, scale=0.088, dt=1)
    a.update(over)
    return L.lib.msgl_prefill_attn(a["out"], a["lse"], a["q"], a["k"], a["v"], a["S"], a["pt"], a["W"],
                                   a["tix"], a["sl"], a["cl"], a["cu"], a["bs"], a["T"], a["me"], a["H"],
                                   a["G"], a["d"], a["ps"], a["scale"], a["dt"], None)


def test_prefill_argument_checks(L):
    assert _prefill(L, T=1) == L.MSGL_INVALID_ARG   # fewer tokens than requests
    assert _prefill(L, me=0) == L.MSGL_INVALID_ARG
    assert _prefill(L, me=11) == L.MSGL_INVALID_ARG
    assert _prefill(L, cl=None) == L.MSGL_INVALID_ARG
    assert _prefill(L, bs=0, T=3) == L.MSGL_INVALID_ARG
    assert _prefill(L, bs=0, T=0) == L.MSGL_OK
    assert _prefill(L, G=3) == L.MSGL_INVALID_ARG


def test_graph_handle_checks(L):
    lib = L.lib
    assert lib.msgl_graph_launch(None, None) == L.MSGL_INVALID_ARG
    lib.msgl_graph_destroy(None)
    h = ctypes.c_void_p()
    st = lib.msgl_decode_graph_create(ctypes.byref(h), FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      FAKE, 64, FAKE, FAKE, 4, 32, 8, 128, 1, 64, 0, 0.1, 1, FAKE, 1 << 20,
                                      None)
    assert st == L.MSGL_INVALID_ARG and "stream" in L.msgl_last_error()


def test_validate_batch(L):
    from paged_kv_attention_slots_amd import workloads as wl

    w = wl.qwen3_8b_decode(page_size=16, bs=5, num_slots=1 << 12, median=100.0, hi=512)
    args = dict(max_seq_len=w.max_seq_len, num_slots=w.num_slots_total, page_size=16)
    L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, w.cached_lens, w.cu_q,
                          out_loc=w.out_loc, dummy_slot=w.dummy_slot, **args)
    p = wl.pad_decode(w, 8)
    L.msgl_validate_batch(p.page_table, p.table_idx, p.seq_lens, p.cached_lens, p.cu_q,
                          out_loc=p.out_loc, dummy_slot=w.dummy_slot, **args)
    with pytest.raises(L.MsglError):  # repeated dummy slot not allowed without naming it
        L.msgl_validate_batch(p.page_table, p.table_idx, p.seq_lens, p.cached_lens, p.cu_q,
                              out_loc=p.out_loc, dummy_slot=-1, **args)
    bad = w.page_table.clone()
    bad[0, 3] += 1  # breaks page contiguity
    with pytest.raises(L.MsglError, match="contiguity"):
        L.msgl_validate_batch(bad, w.table_idx, w.seq_lens, w.cached_lens, w.cu_q, **args)
    sl = w.seq_lens.clone()
    sl[1] = 0
    with pytest.raises(L.MsglError, match="seq_lens"):
        L.msgl_validate_batch(w.page_table, w.table_idx, sl, None, None, **args)
    cu = w.cu_q.clone()
    cu[2] += 1
    with pytest.raises(L.MsglError, match="cu_q"):
        L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, w.cached_lens, cu, **args)
    loc = w.out_loc.clone()
    loc[0] = w.num_slots_total
    with pytest.raises(L.MsglError, match="out_loc"):
        L.msgl_validate_batch(w.page_table, w.table_idx, w.seq_lens, w.cached_lens, w.cu_q,
                              out_loc=loc, **args)
    tix = w.table_idx.clone()
    tix[0] = 99
    with pytest.raises(L.MsglError, match="table_idx"):
        L.msgl_validate_batch(w.page_table, tix, w.seq_lens, None, None, **args)
    pt = w.page_table.clone()
    pt[2, 0] = -5
    with pytest.raises(L.MsglError, match="page_table"):
        L.msgl_validate_batch(pt, w.table_idx, w.seq_lens, None, None, max_seq_len=w.max_seq_len,
                              num_slots=w.num_slots_total, page_size=1)


def test_check_batch_argument_checks(L):
    """msgl_check_batch refuses NULL required pointers, bad scalars and
    out_loc checks it cannot place, before any launch."""
    lib = ctypes.CDLL(L.LIB_PATH)
    f = lib.msgl_check_batch
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.argtypes = [P, I32, I32, P, P, P, P, I32, I32, I64, I32, P, I32, I64, P, P, P]
    FAKE = 4096  # never dereferenced: every call below fails its host checks first
    ok_args = [FAKE, 4, 64, FAKE, FAKE, None, None, 4, 64, 1000, 1, None, 0, -1, FAKE, None, None]

    def call(**kw):
        a = list(ok_args)
        names = ["page_table", "rows", "row_stride", "table_idx", "seq_lens", "cached_lens", "cu_q", "batch",
                 "max_seq_len", "num_slots", "page_size", "out_loc", "num_tokens", "dummy_slot", "result", "seen",
                 "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(page_table=None) == L.MSGL_INVALID_ARG
    assert call(result=None) == L.MSGL_INVALID_ARG and "NULL" in L.msgl_last_error()
    assert call(rows=0) == L.MSGL_INVALID_ARG
    assert call(page_size=0) == L.MSGL_INVALID_ARG
    assert call(num_tokens=-1) == L.MSGL_INVALID_ARG
    assert call(out_loc=FAKE, cached_lens=FAKE, num_tokens=4) == L.MSGL_INVALID_ARG
    assert "cu_q" in L.msgl_last_error()
    assert call(out_loc=FAKE, num_tokens=3) == L.MSGL_INVALID_ARG and "decode" in L.msgl_last_error()
    assert call(num_slots=1 << 31) == L.MSGL_UNSUPPORTED


def test_binding_refuses_host_tensors(L):
    x = torch.zeros(4, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        L.msgl_store_kv(x, x, x[:1], x[:1], torch.zeros(1, dtype=torch.int32))


def test_measurement_probes_exported():
    """The bench's ceiling probes (a separate library, never linked into the
    product) load and reject malformed calls before any launch."""
    from paged_kv_attention_slots_amd import build as _build

    if not os.path.exists(_build.PROBES_PATH):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(_build.PROBES_PATH)
    for n in ("msglp_stream_read", "msglp_gather_heads", "msglp_mfma_loop"):
        assert hasattr(lib, n), n
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.msglp_mfma_loop.argtypes = [I, I, P, I, I, P, P, P]
    lib.msglp_stream_read.argtypes = [P, I64, P, I, P]
    invalid = 1  # hipErrorInvalidValue
    assert lib.msglp_mfma_loop(0, 0, None, 0, 10, None, None, None) == invalid  # no blocks
    assert lib.msglp_mfma_loop(4, 0, None, 1, 10, None, None, None) == invalid  # unknown variant
    assert lib.msglp_mfma_loop(3, 1, None, 1, 10, None, None, None) == invalid  # 16x16x32: 32 columns only
    assert lib.msglp_mfma_loop(0, 0, None, 1, 0, None, None, None) == invalid   # no units
    assert lib.msglp_stream_read(None, 15, None, 1, None) == invalid            # not a multiple of 16
    product = ctypes.CDLL(_build.LIB_PATH)
    assert not hasattr(product, "msglp_mfma_loop") and not hasattr(product, "msglp_stream_read")
