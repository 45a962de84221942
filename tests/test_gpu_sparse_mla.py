"""dsa_sparse_mla_attn on the GPU against the oracle, fed the same indices (rule: outputs
within 1e-5 relative for fp32 and 2e-3 for bf16 per head row; lse likewise per query)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import RTOL, assert_rowwise, binding, check_guards, dev, guarded, guarded_workspace, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402


def _indices(B, n_q, n_kv, top_k, seed, pad=0, bad=0):
    rng = np.random.default_rng(seed)
    idx = np.full((B, n_q, top_k), -1, np.int32)
    for b in range(B):
        for i in range(n_q):
            k = min(top_k - pad, n_kv)
            sel = np.sort(rng.choice(n_kv, k, replace=False)).astype(np.int32)
            idx[b, i, :k] = sel
            if bad:
                idx[b, i, rng.choice(top_k, bad, replace=False)] = n_kv + 5  # out of range: skipped
    return idx


def _run(wl, idx, seed, n_split=0, kv_len=None):
    L = binding()
    inp = workloads.gen_all(wl, seed, parts=("qa", "latent"))
    out = guarded((wl.B, wl.n_q, wl.Hm, wl.d_latent), torch.float32, fill=3.0)
    lse = guarded((wl.B, wl.n_q, wl.Hm), torch.float32, fill=3.0)
    ws = guarded_workspace(L.dsa_sparse_mla_workspace_size(wl.B, wl.n_q, wl.Hm, idx.shape[-1], wl.d_latent, n_split))
    L.dsa_sparse_mla_attn(dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype), dev(idx), out,
                          wl.d_latent, wl.sm_scale, lse=lse, kv_len=dev(np.asarray(kv_len, np.int32)) if kv_len is not None else None,
                          n_split=n_split, workspace=ws)
    check_guards(f"{wl.name} attention")
    o_w, l_w = oracle.sparse_mla(inp["qa"], inp["latent"], idx, wl.sm_scale, wl.d_latent, wl.mla_dtype, kv_len)
    rt = RTOL[wl.mla_dtype]
    assert_rowwise(host(out), o_w, rt, f"{wl.name} out")
    assert_rowwise(host(lse), l_w, rt, f"{wl.name} lse")
    return host(out), host(lse)


def test_tiny_fp32_workload():
    wl = workloads.TINY_FP32
    _run(wl, _indices(1, 1, wl.n_kv, wl.top_k, 0), 0)


DEC = workloads.GLM_DECODE_8K


@pytest.mark.parametrize("Hm,top_k,n_split", [(64, 1, 1), (64, 31, 1), (64, 32, 1), (64, 33, 1), (64, 100, 3),
                                              (16, 300, 2), (48, 256, 1), (64, 2048, 0), (64, 2048, 8),
                                              (32, 513, 5), (48, 256, 4), (16, 300, 1), (32, 100, 1)])
def test_mfma_shapes(Hm, top_k, n_split):
    wl = DEC.scaled(B=2, n_kv=3000, Hm=Hm, top_k=top_k)
    _run(wl, _indices(2, 1, wl.n_kv, top_k, top_k), 1, n_split)


def test_mfma_padding_out_of_range_and_kv_len():
    wl = DEC.scaled(B=3, n_q=2, n_kv=500, top_k=200)
    idx = _indices(3, 2, wl.n_kv, 200, 2, pad=37, bad=9)
    _run(wl, idx, 2, n_split=3, kv_len=[500, 250, 499])


def test_mfma_no_rope():
    wl = DEC.scaled(B=1, n_kv=700, d_rope=0, top_k=128)
    _run(wl, _indices(1, 1, 700, 128, 3), 3, n_split=2)


def test_empty_selection():
    L = binding()
    wl = DEC.scaled(B=1, n_kv=100, top_k=64)
    inp = workloads.gen_all(wl, 4, parts=("qa", "latent"))
    idx = np.full((1, 1, 64), -1, np.int32)
    for n_split in (1, 4):
        out = torch.full((1, 1, 64, 512), 3.0, dtype=torch.float32, device="cuda")
        lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
        L.dsa_sparse_mla_attn(dev(inp["qa"], wl.mla_dtype), dev(inp["latent"], wl.mla_dtype), dev(idx), out,
                              512, wl.sm_scale, lse=lse, n_split=n_split)
        torch.cuda.synchronize()
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("dtype,Hm", [(workloads.F32, 8), (workloads.BF16, 8), (workloads.F32, 20)])
def test_plain_path(dtype, Hm):
    wl = DEC.scaled(B=2, n_kv=400, Hm=Hm, top_k=100, mla_dtype=dtype)
    _run(wl, _indices(2, 1, 400, 100, 5, pad=3), 5, n_split=2)


def test_peaked_softmax():
    # a query aligned with one row makes the softmax nearly one-hot
    L = binding()
    wl = DEC.scaled(B=1, n_kv=300, top_k=64)
    inp = workloads.gen_all(wl, 6, parts=("qa", "latent"))
    lat = oracle.decode(inp["latent"], wl.mla_dtype)
    qa = np.repeat(lat[0, 17][None, None, None, :] * 12.0, 64, axis=2)
    qa_bits = workloads.round_to(qa, wl.mla_dtype)
    rng = np.random.default_rng(6)
    others = rng.choice(np.setdiff1d(np.arange(300), [17]), 63, replace=False)
    idx = np.sort(np.concatenate([others, [17]])).astype(np.int32)[None, None, :]
    out = torch.empty((1, 1, 64, 512), dtype=torch.float32, device="cuda")
    L.dsa_sparse_mla_attn(dev(qa_bits, wl.mla_dtype), dev(inp["latent"], wl.mla_dtype), dev(idx), out, 512,
                          wl.sm_scale)
    torch.cuda.synchronize()
    o_w, _ = oracle.sparse_mla(qa_bits, inp["latent"], idx, wl.sm_scale, 512, wl.mla_dtype)
    assert_rowwise(host(out), o_w, 2e-3, "peaked")


def test_splits_agree():
    wl = DEC.scaled(B=2, n_kv=5000, top_k=2048)
    idx = _indices(2, 1, 5000, 2048, 7)
    a, la = _run(wl, idx, 7, n_split=1)
    b, lb = _run(wl, idx, 7, n_split=16)
    assert_rowwise(b, a, 1e-5, "split 16 vs 1")


def test_deterministic():
    wl = DEC.scaled(B=2, n_kv=5000, top_k=2048)
    idx = _indices(2, 1, 5000, 2048, 8)
    a, _ = _run(wl, idx, 8)
    b, _ = _run(wl, idx, 8)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.fixture
def one_tile_per_step():
    """The kernel variant taking one 16-row tile between barriers (the automatic choice takes
    two, or three for parts of 1024 slots or more)."""
    L = binding()
    L.dsa_set_tuning("mla_tiles_per_step", 1)
    yield
    L.dsa_set_tuning("mla_tiles_per_step", 0)


@pytest.fixture
def three_tiles_per_step():
    """The kernel variant taking three 16-row tiles between barriers (a 6-stage ring in which a
    step refills its own stages), forced on every shape."""
    L = binding()
    L.dsa_set_tuning("mla_tiles_per_step", 3)
    yield
    L.dsa_set_tuning("mla_tiles_per_step", 0)


@pytest.mark.parametrize("Hm,top_k,n_split,d_rope", [(64, 1, 1, 64), (64, 17, 1, 64), (64, 32, 1, 64),
                                                     (64, 33, 1, 64), (64, 100, 3, 64), (16, 300, 2, 64),
                                                     (48, 256, 4, 64), (64, 2048, 0, 64), (64, 2048, 8, 64),
                                                     (32, 513, 5, 64), (64, 2051, 0, 0), (64, 2048, 1, 64)])
def test_one_tile_per_step(one_tile_per_step, Hm, top_k, n_split, d_rope):
    """The shapes of the MFMA tests with one 16-row tile between barriers (the default takes two:
    one softmax update and one probability buffer per 32 rows, odd tile counts ending with a
    padding tile, which the default-path tests above cover)."""
    wl = DEC.scaled(B=2, n_kv=3000, Hm=Hm, top_k=top_k, d_rope=d_rope)
    _run(wl, _indices(2, 1, wl.n_kv, top_k, top_k + 11), 1, n_split)


@pytest.mark.parametrize("Hm,top_k,n_split,d_rope", [(64, 1, 1, 64), (64, 47, 1, 64), (64, 48, 1, 64),
                                                     (64, 49, 1, 64), (64, 95, 1, 64), (64, 97, 2, 64),
                                                     (16, 300, 2, 64), (48, 256, 4, 64), (64, 2048, 0, 64),
                                                     (64, 2048, 8, 64), (32, 513, 5, 64), (64, 2051, 0, 0),
                                                     (64, 2048, 1, 64), (64, 288, 1, 64), (32, 700, 1, 0),
                                                     (16, 1100, 1, 64)])
def test_three_tiles_per_step(three_tiles_per_step, Hm, top_k, n_split, d_rope):
    """The MFMA shapes with three 16-row tiles between barriers: slot counts below one step,
    at and around a step's 48 rows, ragged parts, the ring's two-step prologue with one or two
    steps in all, 32-head rows and 512-wide rows."""
    wl = DEC.scaled(B=2, n_kv=3000, Hm=Hm, top_k=top_k, d_rope=d_rope)
    _run(wl, _indices(2, 1, wl.n_kv, top_k, top_k + 13), 1, n_split)


def test_three_tiles_per_step_padding_kv_len_and_peaks(three_tiles_per_step):
    wl = DEC.scaled(B=3, n_q=2, n_kv=500, top_k=200)
    _run(wl, _indices(3, 2, wl.n_kv, 200, 2, pad=37, bad=9), 2, n_split=3, kv_len=[500, 250, 499])
    test_peaked_softmax()
    test_empty_selection()
    wl = DEC.scaled(B=2, n_kv=5000, top_k=2048)
    idx = _indices(2, 1, 5000, 2048, 7)
    a, _ = _run(wl, idx, 7, n_split=1)
    b, _ = _run(wl, idx, 7, n_split=16)
    assert_rowwise(b, a, 1e-5, "three tiles per step: split 16 vs 1")


def test_one_tile_per_step_padding_kv_len_and_peaks(one_tile_per_step):
    wl = DEC.scaled(B=3, n_q=2, n_kv=500, top_k=200)
    _run(wl, _indices(3, 2, wl.n_kv, 200, 2, pad=37, bad=9), 2, n_split=3, kv_len=[500, 250, 499])
    test_peaked_softmax()
    test_empty_selection()
    wl = DEC.scaled(B=2, n_kv=5000, top_k=2048)
    idx = _indices(2, 1, 5000, 2048, 7)
    a, _ = _run(wl, idx, 7, n_split=1)
    b, _ = _run(wl, idx, 7, n_split=16)
    assert_rowwise(b, a, 1e-5, "one tile per step: split 16 vs 1")


@pytest.fixture(params=[1, 2], ids=["heads_together", "heads_split"])
def head_split(request):
    """64 heads in one workgroup row, or as two 32-head rows sharing the query's selection (the
    automatic choice splits when 64-head rows would fill at most half of the chip, as in most
    small cases above)."""
    L = binding()
    L.dsa_set_tuning("mla_head_split", request.param)
    yield request.param
    L.dsa_set_tuning("mla_head_split", 0)


@pytest.mark.parametrize("B,top_k,n_split,d_rope", [(2, 2048, 8, 64), (3, 100, 3, 64), (2, 2051, 0, 0),
                                                    (2, 33, 1, 64), (20, 700, 8, 64)])
def test_head_split_forced(head_split, B, top_k, n_split, d_rope):
    wl = DEC.scaled(B=B, n_kv=3000, top_k=top_k, d_rope=d_rope)
    _run(wl, _indices(B, 1, wl.n_kv, top_k, top_k + 5, pad=3), 9, n_split, kv_len=[3000 - 7 * b for b in range(B)])
