"""dsa_index_score on the GPU against the oracle (rule: scores within 1e-5 relative for
fp32 and 2e-3 for bf16/f16 per score row, -inf pattern identical)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import RTOL, assert_rowwise, binding, check_guards, dev, guarded, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _run(wl, seed, kv_len=None, q_pos=None, scale=None):
    L = binding()
    inp = workloads.gen_all(wl, seed, parts=("q", "k", "w"))
    kv = inp["kv_len"] if kv_len is None else np.asarray(kv_len, np.int32)
    qp = q_pos
    if qp is None and wl.q_pos_start is not None:
        qp = inp["q_pos"]
    sc = wl.scale if scale is None else scale
    out = guarded((wl.B, wl.n_q, wl.n_kv), torch.float32, fill=7.0)
    L.dsa_index_score(dev(inp["q"], wl.idx_dtype), dev(inp["k"], wl.idx_dtype), dev(inp["w"]), out,
                      kv_len=dev(kv) if kv_len is not None else None,
                      q_pos=dev(np.asarray(qp, np.int32)) if qp is not None else None, scale=sc)
    check_guards(f"{wl.name} scores")
    want = oracle.index_score(inp["q"], inp["k"], inp["w"], kv, qp, sc, wl.idx_dtype, wl.idx_dtype)
    assert_rowwise(host(out), want, RTOL[wl.idx_dtype], wl.name)
    return host(out), want


def test_tiny_fp32_workload():
    _run(workloads.TINY_FP32, 0)


DEC = workloads.GLM_DECODE_8K


@pytest.mark.parametrize("B,n_kv,H", [(1, 1, 32), (1, 63, 32), (2, 64, 4), (1, 65, 1), (3, 255, 32),
                                      (1, 256, 16), (2, 1000, 32), (1, 5000, 32), (2, 1025, 17)])
def test_decode_bf16_shapes(B, n_kv, H):
    _run(DEC.scaled(B=B, n_kv=n_kv, H=H), 1)


@pytest.mark.parametrize("cpw", [1, 2, 4, 8])
def test_decode_chunks_per_wave(cpw):
    """Every unrolled variant of the decode kernel: ragged kv_len (a chunk straddles the end
    of the scored range, whole chunks lie past it), n_kv not a multiple of a block's keys
    (waves of the last block run past n_kv), a second query per sequence."""
    L = binding()
    L.dsa_set_tuning("score_chunks_per_wave", cpw)
    try:
        _run(DEC.scaled(B=3, n_kv=5000), 5, kv_len=[5000, 3001, 70])
        _run(DEC.scaled(B=2, n_q=2, n_kv=2113), 6, kv_len=[2113, 1500])
        _run(workloads.LONG_DECODE_128K.scaled(B=2, n_kv=4099), 7)
    finally:
        L.dsa_set_tuning("score_chunks_per_wave", 0)


@pytest.mark.parametrize("B,n_kv", [(1, 77), (2, 2100)])
def test_decode_f16(B, n_kv):
    _run(workloads.LONG_DECODE_128K.scaled(B=B, n_kv=n_kv), 2)


def test_decode_ragged_kv_len_and_scale():
    _run(DEC.scaled(B=3, n_kv=300), 3, kv_len=[300, 129, 1], scale=0.5)


def test_decode_two_queries_per_sequence():
    wl = DEC.scaled(B=2, n_q=3, n_kv=500)
    _run(wl, 4, kv_len=[500, 333])


@pytest.mark.parametrize("n_q,n_kv,start", [(8, 700, 692), (13, 700, 687), (40, 700, 300), (64, 2000, 1936),
                                            (9, 130, 0)])
def test_prefill_causal_bf16(n_q, n_kv, start):
    _run(DEC.scaled(n_q=n_q, n_kv=n_kv, q_pos_start=start), 5)


@pytest.mark.parametrize("waves", [4, 8])
def test_prefill_waves_per_block(waves):
    """Each workgroup shape of the prefill kernel: a query count that leaves the last block
    partly empty, causal limits inside and across tiles, a second sequence."""
    L = binding()
    L.dsa_set_tuning("score_prefill_waves", waves)
    try:
        _run(DEC.scaled(B=2, n_q=45, n_kv=1100, q_pos_start=1100 - 45 - 300), 10)
        _run(DEC.scaled(n_q=33, n_kv=700, q_pos_start=0), 11)
    finally:
        L.dsa_set_tuning("score_prefill_waves", 0)


def test_prefill_kv_len_shorter_than_cache():
    wl = DEC.scaled(B=2, n_q=16, n_kv=400, q_pos_start=380)
    _run(wl, 6, kv_len=[390, 200])


@pytest.mark.parametrize("H,D", [(8, 64), (40, 128), (3, 96)])
def test_plain_path_16bit(H, D):
    _run(DEC.scaled(B=2, n_kv=333, H=H, D=D, rotate=False), 7)


def test_chunked_prefill_shape_small():
    # the chunked-prefill workload's structure at a fraction of its size
    wl = workloads.CHUNKED_PREFILL_16K.scaled(n_q=96, n_kv=1024, q_pos_start=1024 - 96 - 200)
    _run(wl, 8)


def test_deterministic():
    wl = DEC.scaled(B=2, n_kv=4099)
    a, _ = _run(wl, 9)
    b, _ = _run(wl, 9)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _run_sink(wl, seed, sink_start, n_sink, kv_len=None):
    L = binding()
    inp = workloads.gen_all(wl, seed, parts=("q", "k", "w"))
    kv = inp["kv_len"] if kv_len is None else np.asarray(kv_len, np.int32)
    qp = inp["q_pos"] if wl.q_pos_start is not None else None
    out = guarded((wl.B, wl.n_q, wl.n_kv), torch.float32, fill=7.0)
    L.dsa_index_score(dev(inp["q"], wl.idx_dtype), dev(inp["k"], wl.idx_dtype), dev(inp["w"]), out,
                      kv_len=dev(kv) if kv_len is not None else None,
                      q_pos=dev(np.asarray(qp, np.int32)) if qp is not None else None, scale=wl.scale,
                      n_sink=n_sink, sink_start=dev(np.asarray(sink_start, np.int32)) if sink_start is not None else None)
    check_guards(f"{wl.name} scores with sink")
    want = oracle.index_score_sink(inp["q"], inp["k"], inp["w"], kv, qp, wl.scale, wl.idx_dtype, wl.idx_dtype,
                                   sink_start, n_sink, 1e20)
    got = host(out)
    boosted = want > 1e19
    assert boosted.any()
    assert np.array_equal(got[boosted], want[boosted]), "boosted scores"
    assert np.array_equal(got > 1e19, boosted), "boosted positions"
    g2, w2 = got.copy(), want.copy()
    g2[boosted] = 0.0
    w2[boosted] = 0.0
    assert_rowwise(g2, w2, RTOL[wl.idx_dtype], wl.name + " with sink")
    # the sink survives top-k (n_sink <= top_k)
    rows = wl.B * wl.n_q
    k_sel = min(wl.top_k, 16)
    idx = torch.empty((rows, k_sel), dtype=torch.int32, device="cuda")
    L.dsa_topk(out.view(rows, wl.n_kv), idx, k_sel)
    sel = host(idx).reshape(wl.B, wl.n_q, k_sel)
    for b in range(wl.B):
        for i in range(wl.n_q):
            must = set(np.nonzero(boosted[b, i])[0].tolist())
            assert must <= set(sel[b, i].tolist()), (b, i)


def test_sink_decode_mfma():
    _run_sink(DEC.scaled(B=3, n_kv=3000), 21, [0, 100, 2990], 4, kv_len=[3000, 2000, 2995])


def test_sink_default_start_and_f16():
    _run_sink(workloads.LONG_DECODE_128K.scaled(B=2, n_kv=1500), 22, None, 2)


def test_sink_prefill():
    _run_sink(DEC.scaled(B=2, n_q=20, n_kv=700, q_pos_start=650), 23, [0, 640], 4)


def test_sink_plain_fp32():
    _run_sink(workloads.TINY_FP32.scaled(B=2), 24, [3, 0], 2)
