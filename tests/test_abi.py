"""The C ABI without a GPU: the library loads, exports what include/dsa.h declares, and
rejects bad arguments on the host before anything is launched (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB = os.path.join(ROOT, "sparse_attention_10_amd", "libdsa.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_WS, E_UNSUP, E_HIP = 0, -1, -2, -3, -4, -5, -6
FAKE = 0x100000  # a non-NULL pointer that validation must never dereference


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dsa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    from sparse_attention_10_amd import dsa
    return dsa.lib


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_attn", "dsa_topk_workspace_size",
              "dsa_sparse_mla_workspace_size", "dsa_status_string", "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dsa_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    # nothing else with the dsa_ prefix leaks out unexported in the header
    assert exported <= set(names), exported - set(names)


def test_binding_lists_every_export(lib):
    from sparse_attention_10_amd import dsa
    assert set(dsa.EXPORTED) == set(declared_functions())


def test_status_strings(lib):
    for s in (OK, E_NULL, E_SHAPE, E_DTYPE, E_WS, E_UNSUP, E_HIP):
        assert lib.dsa_status_string(s).startswith(b"DSA_")
    assert lib.dsa_version() >= 100


def _score(lib, q=FAKE, k=FAKE, w=FAKE, s=FAKE, B=1, n_q=1, H=32, D=128, n_kv=64, qd=1, kd=1):
    return lib.dsa_index_score(q, k, w, None, None, s, B, n_q, H, D, n_kv, qd, kd, 1.0, None)


def test_index_score_rejects_on_host(lib):
    assert _score(lib, q=None) == E_NULL
    assert _score(lib, s=None) == E_NULL
    assert b"non-NULL" in lib.dsa_last_error()
    for kw in ({"B": 0}, {"n_q": 0}, {"H": 0}, {"D": 0}, {"n_kv": 0}, {"n_kv": -5}):
        assert _score(lib, **kw) == E_SHAPE, kw
    assert _score(lib, qd=7, kd=7) == E_DTYPE
    assert _score(lib, qd=1, kd=2) == E_DTYPE
    assert _score(lib, q=FAKE + 2) == E_UNSUP          # MFMA path needs 16-byte alignment
    assert _score(lib, H=200, D=100, qd=0, kd=0) == E_UNSUP  # plain path limit H*D <= 16384


def test_topk_rejects_on_host(lib):
    assert lib.dsa_topk(None, FAKE, 1, 10, 2, None, 0, None) == E_NULL
    assert lib.dsa_topk(FAKE, FAKE, 0, 10, 2, None, 0, None) == E_SHAPE
    assert lib.dsa_topk(FAKE, FAKE, 1, 10, 0, None, 0, None) == E_SHAPE
    need = lib.dsa_topk_workspace_size(8, 131072, 2048)
    assert need > 0
    assert lib.dsa_topk(FAKE, FAKE, 8, 131072, 2048, None, 0, None) == E_WS
    assert lib.dsa_topk(FAKE, FAKE, 8, 131072, 2048, FAKE, need - 1, None) == E_WS
    assert b"workspace" in lib.dsa_last_error()


def test_topk_workspace_size_monotone(lib):
    f = lib.dsa_topk_workspace_size
    assert f(0, 100, 4) == 0 and f(1, 100, 0) == 0
    prev = 0
    for rows in (1, 2, 8, 32, 256):
        cur = f(rows, 131072, 2048)
        assert cur >= prev
        prev = cur
    assert f(8, 131072, 1024) <= f(8, 131072, 2048)


def _mla(lib, qa=FAKE, lat=FAKE, idx=FAKE, out=FAKE, B=1, n_q=1, Hm=64, n_kv=128, top_k=64, dl=512,
         dr=64, dtype=1, n_split=1, ws=None, wsb=0):
    return lib.dsa_sparse_mla_attn(qa, lat, idx, None, out, None, B, n_q, Hm, n_kv, top_k, dl, dr,
                                   0.0625, dtype, n_split, ws, wsb, None)


def test_sparse_mla_rejects_on_host(lib):
    assert _mla(lib, qa=None) == E_NULL
    assert _mla(lib, idx=None) == E_NULL
    for kw in ({"B": 0}, {"Hm": 0}, {"top_k": 0}, {"dl": 0}, {"dr": -1}, {"n_kv": 0}):
        assert _mla(lib, **kw) == E_SHAPE, kw
    assert _mla(lib, dtype=2) == E_DTYPE
    assert _mla(lib, dtype=9) == E_DTYPE
    assert _mla(lib, top_k=4096, n_split=1) == E_UNSUP           # > 2048 slots per part on MFMA
    assert _mla(lib, lat=FAKE + 4) == E_UNSUP                   # alignment
    assert _mla(lib, Hm=8, dl=1000, dr=100, dtype=0) == E_UNSUP  # plain path limit
    need = lib.dsa_sparse_mla_workspace_size(1, 1, 64, 2048, 512, 8)
    assert need > 0
    assert _mla(lib, top_k=2048, n_split=8) == E_WS
    assert _mla(lib, top_k=2048, n_split=8, ws=FAKE, wsb=need - 1) == E_WS


def test_sparse_mla_workspace_size(lib):
    f = lib.dsa_sparse_mla_workspace_size
    assert f(4, 1, 64, 2048, 512, 1) == 0
    prev = 0
    for s in (2, 3, 8, 16):
        cur = f(4, 1, 64, 2048, 512, s)
        assert cur > prev
        prev = cur
    # n_split <= 0 resolves to the automatic count
    auto = lib.dsa_sparse_mla_num_splits(32, 1, 2048)
    assert auto >= 1
    assert f(32, 1, 64, 2048, 512, 0) == f(32, 1, 64, 2048, 512, auto)


def test_auto_splits_fit_one_round_of_workgroups(lib):
    """The automatic part count never asks for more than one workgroup per CU (256) beyond what
    the selection's length forces, and keeps parts of at least 128 slots when it splits."""
    f = lib.dsa_sparse_mla_num_splits
    for top_k in (64, 2048, 2051):
        for rows in range(1, 300):
            s = f(rows, 1, top_k)
            assert s >= 1
            forced = -(-top_k // 2048)  # one part holds at most 2048 slots
            assert rows * s <= 256 or s == forced, (rows, top_k, s)
            assert s == 1 or top_k // s >= 16, (rows, top_k, s)
    assert f(32, 1, 2048) == 6 and f(64, 1, 2048) == 4 and f(8, 1, 2048) == 16
    assert f(1, 4096, 2048) == 1  # a prefill chunk: one part per query


def test_tuning_switch(lib):
    assert lib.dsa_set_tuning(b"topk_path", 2) == OK
    assert lib.dsa_set_tuning(b"topk_path", 0) == OK
    assert lib.dsa_set_tuning(b"topk_path", 3) == OK
    assert lib.dsa_set_tuning(b"topk_path", 4) == E_SHAPE
    assert lib.dsa_set_tuning(b"score_chunks_per_wave", 4) == OK
    assert lib.dsa_set_tuning(b"score_chunks_per_wave", 0) == OK
    assert lib.dsa_set_tuning(b"score_chunks_per_wave", 65) == E_SHAPE
    assert lib.dsa_set_tuning(b"score_chunks_per_wave", -1) == E_SHAPE
    for v in (1, 2, 3, 0):
        assert lib.dsa_set_tuning(b"mla_tiles_per_step", v) == OK
    assert lib.dsa_set_tuning(b"mla_tiles_per_step", 4) == E_SHAPE
    assert lib.dsa_set_tuning(b"mla_tiles_per_step", -1) == E_SHAPE
    for v in (1, 2, 0):
        assert lib.dsa_set_tuning(b"mla_head_split", v) == OK
    assert lib.dsa_set_tuning(b"mla_head_split", 3) == E_SHAPE
    for v in (4, 8, 0):
        assert lib.dsa_set_tuning(b"score_prefill_waves", v) == OK
    for v in (1, 2, 12, 16, -4):
        assert lib.dsa_set_tuning(b"score_prefill_waves", v) == E_SHAPE
    for v in (256, 512, 1024, 0):
        assert lib.dsa_set_tuning(b"topk_cand_block", v) == OK
    for v in (128, 2048, -1):
        assert lib.dsa_set_tuning(b"topk_cand_block", v) == E_SHAPE
    assert lib.dsa_set_tuning(b"no_such_key", 1) == E_SHAPE
    assert lib.dsa_set_tuning(None, 1) == E_NULL


def test_last_error_is_per_thread(lib):
    import threading
    assert _score(lib, q=None) == E_NULL
    seen = {}

    def other():
        seen["err"] = lib.dsa_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["err"] == b""
    assert lib.dsa_last_error() != b""


def _prep(lib, q_in=FAKE, k_in=FAKE, lat=None, pos=FAKE, q_out=FAKE, k_cache=FAKE, lat_cache=None,
          B=1, n_new=1, H=32, n_kv=64, row_bytes=1152, od=1, base=10000.0, had=1):
    return lib.dsa_indexer_prep(q_in, k_in, lat, pos, q_out, k_cache, lat_cache, B, n_new, H, n_kv,
                                row_bytes, od, base, had, None)


def test_indexer_prep_rejects_on_host(lib):
    assert _prep(lib, pos=None) == E_NULL
    assert _prep(lib, q_in=None, k_in=None) == E_NULL               # nothing to do
    assert _prep(lib, q_out=None) == E_NULL                         # unpaired
    assert _prep(lib, k_cache=None) == E_NULL
    assert _prep(lib, lat=FAKE) == E_NULL                           # latent without its cache
    for kw in ({"B": 0}, {"n_new": 0}, {"H": 0}, {"n_kv": 0}):
        assert _prep(lib, **kw) == E_SHAPE, kw
    assert _prep(lib, lat=FAKE, lat_cache=FAKE, row_bytes=1000) == E_SHAPE
    assert _prep(lib, od=9) == E_DTYPE
    for base in (0.0, -1.0, float("inf"), float("nan")):
        assert _prep(lib, base=base) == E_SHAPE, base
    assert _prep(lib, k_cache=FAKE + 8) == E_UNSUP


def test_index_score_sink_rejects_on_host(lib):
    def call(n_sink=2, boost=1e20, q=FAKE):
        return lib.dsa_index_score_sink(q, FAKE, FAKE, None, None, None, n_sink, boost, FAKE, 1, 1, 32, 128, 64,
                                        1, 1, 1.0, None)
    assert call(n_sink=-1) == E_SHAPE
    assert call(boost=float("inf")) == E_SHAPE
    assert call(boost=float("nan")) == E_SHAPE
    assert call(q=None) == E_NULL
    assert b"dsa_index_score_sink" in lib.dsa_last_error()


def test_indexshare_layer_map(lib):
    # GLM-5.2: 21 full and 57 shared layers among 78 (the IndexShare sub-commit's counts)
    full = [l for l in range(78) if lib.dsa_layer_computes_topk(l) == 1]
    assert len(full) == 21 and 78 - len(full) == 57
    assert full[:3] == [0, 1, 2]
    for l in range(200):
        src = lib.dsa_topk_source_layer(l)
        assert lib.dsa_layer_computes_topk(src) == 1
        assert src <= l
        # no full layer lies strictly between the source and the layer
        assert all(lib.dsa_layer_computes_topk(m) == 0 for m in range(src + 1, l + 1))
    assert lib.dsa_layer_computes_topk(-1) == E_SHAPE
    assert lib.dsa_topk_source_layer(-3) == E_SHAPE


def _compress(lib, packed=FAKE, stride=257, rdt=2, ape=FAKE, pooled=FAKE, odt=2, B=2, n_kv=64, D=128, kpool=4,
              p0=0, p1=16):
    return lib.dsa_kpool_compress(packed, stride, rdt, ape, pooled, odt, B, n_kv, D, kpool, p0, p1, None)


def test_kpool_compress_validation(lib):
    assert _compress(lib, packed=None) == E_NULL
    assert _compress(lib, ape=None) == E_NULL
    assert _compress(lib, pooled=None) == E_NULL
    assert _compress(lib, stride=256) == E_SHAPE            # no room for the valid column
    assert _compress(lib, kpool=0) == E_SHAPE
    assert _compress(lib, kpool=9) == E_SHAPE
    assert _compress(lib, p1=17) == E_SHAPE                 # past the 16 complete pools
    assert _compress(lib, p0=5, p1=4) == E_SHAPE
    assert _compress(lib, p0=-1) == E_SHAPE
    assert _compress(lib, rdt=7) == E_DTYPE
    assert _compress(lib, odt=-1) == E_DTYPE
    assert _compress(lib, p0=3, p1=3) == OK                 # empty range: nothing launched
    # one thread per (pool, dim): at most 2^31 - 1 of them per call
    assert _compress(lib, n_kv=1 << 26, D=4096, stride=8193, B=1, p1=(1 << 24)) == E_SHAPE


def test_kpool_score_and_expand_validation(lib):
    f = lib.dsa_kpool_index_score
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 1, 1, 32, 128, 100, 0, 1, 1, 1.0, None) == E_SHAPE
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 1, 1, 32, 128, 100, 9, 1, 1, 1.0, None) == E_SHAPE
    assert f(None, FAKE, FAKE, None, None, FAKE, 1, 1, 32, 128, 100, 4, 1, 1, 1.0, None) == E_NULL
    assert f(FAKE, FAKE, FAKE, None, None, FAKE, 1, 1, 32, 128, 100, 4, 1, 2, 1.0, None) == E_DTYPE
    g = lib.dsa_kpool_expand
    assert g(None, FAKE, 257, 2, 128, None, None, FAKE, 1, 1, 64, 4, 4, None) == E_NULL
    assert g(FAKE, FAKE, 257, 2, 128, None, None, None, 1, 1, 64, 4, 4, None) == E_NULL
    assert g(FAKE, FAKE, 256, 2, 128, None, None, FAKE, 1, 1, 64, 4, 4, None) == E_SHAPE
    assert g(FAKE, FAKE, 257, 2, 128, None, None, FAKE, 1, 1, 64, 0, 4, None) == E_SHAPE
    assert g(FAKE, FAKE, 257, 2, 128, None, None, FAKE, 1, 1, 64, 4, 0, None) == E_SHAPE
    assert g(FAKE, FAKE, 257, 2, 128, None, None, FAKE, 300, 300, 64, 4, 4, None) == E_SHAPE
    assert g(FAKE, FAKE, 257, 5, 128, None, None, FAKE, 1, 1, 64, 4, 4, None) == E_DTYPE


def _kpmla(lib, **kw):
    a = dict(q=FAKE, lat=FAKE, pidx=FAKE, packed=FAKE, stride=257, rdt=2, D=128, kv_len=None, q_pos=None,
             out=FAKE, lse=None, B=2, n_q=1, Hm=64, n_kv=4096, top_pools=512, kpool=4, dl=512, dr=0, sm=0.0625,
             dt=1, ns=8, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.dsa_kpool_sparse_mla_attn(a["q"], a["lat"], a["pidx"], a["packed"], a["stride"], a["rdt"], a["D"],
                                         a["kv_len"], a["q_pos"], a["out"], a["lse"], a["B"], a["n_q"], a["Hm"],
                                         a["n_kv"], a["top_pools"], a["kpool"], a["dl"], a["dr"], a["sm"], a["dt"],
                                         a["ns"], a["ws"], a["wsb"], None)


def test_kpool_sparse_mla_validation(lib):
    for k in ("q", "lat", "pidx", "packed", "out"):
        assert _kpmla(lib, **{k: None}) == E_NULL, k
    assert _kpmla(lib, stride=256) == E_SHAPE           # no room for the valid column
    assert _kpmla(lib, kpool=0) == E_SHAPE
    assert _kpmla(lib, kpool=9) == E_SHAPE
    assert _kpmla(lib, top_pools=0) == E_SHAPE
    assert _kpmla(lib, rdt=7) == E_DTYPE
    assert _kpmla(lib, dt=2) == E_DTYPE                 # f16 attention
    assert _kpmla(lib, dt=0) == E_UNSUP                 # fp32 attention: the two calls instead
    assert _kpmla(lib, Hm=8) == E_UNSUP
    assert _kpmla(lib, dr=32) == E_UNSUP
    assert _kpmla(lib, ns=1) == E_UNSUP                 # 2051 slots in one part
    assert _kpmla(lib, q=FAKE + 8) == E_UNSUP           # 16-byte alignment
    assert _kpmla(lib, packed=FAKE + 1) == E_UNSUP      # element alignment of the packed rows
    assert _kpmla(lib, ws=None) == E_WS
    need = lib.dsa_sparse_mla_workspace_size(2, 1, 64, 4 * 512 + 3, 512, 8)
    assert need > 0
    assert _kpmla(lib, wsb=need - 1) == E_WS


def test_launch_grid_limits_rejected_on_host(lib):
    # decode / plain score kernels: B * n_q on the grid's y dimension
    assert _score(lib, B=65536, n_q=1) == E_UNSUP
    assert b"launch grid" in lib.dsa_last_error()
    assert _score(lib, B=16384, n_q=4) == E_UNSUP
    assert _score(lib, B=70000, n_q=1, qd=0, kd=0) == E_UNSUP         # plain kernel
    # prefill kernel (16-bit, D = 128, n_q >= 8): B on the grid's z dimension
    # (only rejected calls here: an accepted one would launch on the fake pointers)
    assert _score(lib, B=65536, n_q=8) == E_UNSUP
    # plain MLA kernel: B * n_q on the grid's y dimension
    assert _mla(lib, B=65536, Hm=8, dl=64, dr=0, dtype=0, top_k=16) == E_UNSUP
    assert b"launch grid" in lib.dsa_last_error()


def test_tuning_is_read_once_per_call_source():
    """The head-split switch is read once per attention call, so the kernel and its merge
    always agree on the layout (a source check: the switch's only reads are at the call's
    start)."""
    src = open(os.path.join(ROOT, "sparse_attention_10_amd", "csrc", "sparse_mla.hip")).read()
    assert src.count("g_mla_head_split.load") == 1
    assert src.count("g_mla_tiles_per_step.load") == 1
    assert "mla_head_split(Hm, rows, n_split)" not in src


def test_topk_noalloc_rejects_on_host(lib):
    assert lib.dsa_topk_noalloc(None, FAKE, 1, 10, 2, None) == E_NULL
    assert lib.dsa_topk_noalloc(FAKE, FAKE, 0, 10, 2, None) == E_SHAPE
    assert lib.dsa_topk_noalloc(FAKE, FAKE, 70000, 10, 2, None) == E_SHAPE
    # a shape whose workspace exceeds the static scratch array
    assert lib.dsa_topk_workspace_size(256, 1 << 20, 2048) > (16 << 20)
    assert lib.dsa_topk_noalloc(FAKE, FAKE, 256, 1 << 20, 2048, None) == E_UNSUP
    assert b"static array" in lib.dsa_last_error()
