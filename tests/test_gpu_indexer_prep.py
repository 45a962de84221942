"""dsa_indexer_prep on the GPU against the oracle (rope, Hadamard rotation, cache append).

Rule for the 16-bit outputs: per element, |g - o| <= one unit in the last place of the
storage format at o, plus 1e-5 * max |o| of the row. The oracle rounds its float64 value
to the storage format; the kernel rounds its float32 value, so the two may land on
neighbouring codes, and the second term covers the float32 error of the 128-term rotation
where it cancels (at most about 128 * 2^-24 of the row's largest input). fp32 outputs:
row-normwise 1e-5. Cache rows not named by a position must keep their bits; latent rows are
copied bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import binding, dev, host

pytestmark = pytest.mark.gpu
import torch  # noqa: E402

F32, BF16, F16 = workloads.F32, workloads.BF16, workloads.F16
TORCH = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}


def _as_f64(bits, dtype):
    return oracle.decode(bits, dtype)


def _ulp(o64, dtype):
    """Spacing of the storage format at |o| (normal range; the subnormal spacing below)."""
    mant = 7 if dtype == BF16 else 10
    emin = -126 if dtype == BF16 else -14
    e = np.floor(np.log2(np.maximum(np.abs(o64), 2.0 ** emin)))
    return 2.0 ** (e - mant)


def assert_storage_close(got, want, dtype, what):
    g = _as_f64(got, dtype).reshape(-1, 128) if dtype != F32 else np.asarray(got, np.float64).reshape(-1, 128)
    o = _as_f64(want, dtype).reshape(-1, 128) if dtype != F32 else np.asarray(want, np.float64).reshape(-1, 128)
    row_max = np.abs(o).max(axis=1, keepdims=True)
    if dtype == F32:
        tol = 1e-5 * row_max
    else:
        tol = _ulp(o, dtype) + 1e-5 * row_max
    err = np.abs(g - o)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{what}: {len(bad)} elements off, first at {tuple(bad[0])}: "
                           f"{g[tuple(bad[0])]!r} vs {o[tuple(bad[0])]!r}")


def _run(B, n_new, H, n_kv, pos, out_dtype, seed, hadamard=True, base=10000.0, with_latent=True, q=True, k=True):
    L = binding()
    rng = np.random.default_rng(seed)
    q_in = (rng.standard_normal((B, n_new, H, 128)) / np.sqrt(128)).astype(np.float32)
    k_in = (rng.standard_normal((B, n_new, 128)) / np.sqrt(128)).astype(np.float32)
    lat_in = rng.integers(0, 1 << 16, size=(B, n_new, 576), dtype=np.uint16)
    pos = np.asarray(pos, np.int32).reshape(B, n_new)
    k0 = rng.standard_normal((B, n_kv, 128)).astype(np.float32)
    k0 = oracle.encode(k0, out_dtype)
    lat0 = rng.integers(0, 1 << 16, size=(B, n_kv, 576), dtype=np.uint16)

    q_out = torch.full((B, n_new, H, 128), 5.0, dtype=TORCH[out_dtype], device="cuda")
    k_cache = dev(k0, out_dtype)
    lat_cache = dev(lat0, BF16)
    L.dsa_indexer_prep(dev(pos), q_in=dev(q_in) if q else None, q_out=q_out if q else None,
                       k_in=dev(k_in) if k else None, k_cache=k_cache if k else None,
                       latent_in=dev(lat_in, BF16) if with_latent else None,
                       latent_cache=lat_cache if with_latent else None, rope_base=base, hadamard=hadamard)
    torch.cuda.synchronize()

    qw, kw = oracle.indexer_prep(q_in if q else None, k_in if k else None, pos, base, out_dtype, hadamard)
    def bits(t):
        a = host(t.view(torch.int16) if t.dtype != torch.float32 else t)
        return a.view(np.uint16) if t.dtype != torch.float32 else a
    if q:
        assert_storage_close(bits(q_out), qw, out_dtype, "q_out")
    kg = bits(k_cache)
    k_want_rows = oracle.cache_append(np.zeros((B, n_kv), np.int8), np.ones((B, n_new), np.int8), pos)
    written = k_want_rows.astype(bool) if k else np.zeros((B, n_kv), bool)
    assert np.array_equal(kg[~written], k0[~written]), "k_cache rows without a position changed"
    if k and written.any():
        k_want = oracle.cache_append(k0, kw, pos)
        assert_storage_close(kg[written], k_want[written], out_dtype, "k_cache rows")
    lg = host(lat_cache.view(torch.int16)).view(np.uint16)
    lat_want = oracle.cache_append(lat0, lat_in, pos) if with_latent else lat0
    assert np.array_equal(lg, lat_want), "latent cache"


@pytest.mark.parametrize("out_dtype", [BF16, F16, F32])
def test_small_mixed_positions(out_dtype):
    # positions: start, middle, last row, large ones, and two outside the cache
    pos = [[0, 17, 49], [131071, -1, 50]]
    _run(2, 3, 32, 50, pos, out_dtype, seed=1)


def test_no_rotation_and_other_heads():
    _run(2, 5, 7, 64, [[0, 1, 2, 3, 63], [10, 20, 30, 40, 50]], BF16, seed=2, hadamard=False)


def test_rope_base_and_huge_positions():
    _run(1, 4, 3, 8, [[1 << 20, (1 << 31) - 1, 7, 3]], F16, seed=3, base=500000.0)


def test_keys_only_and_queries_only():
    _run(3, 2, 4, 16, [[0, 15], [3, 4], [15, 0]], BF16, seed=4, q=False, with_latent=False)
    _run(3, 2, 4, 16, [[0, 15], [3, 4], [15, 0]], BF16, seed=5, k=False)


def test_ragged_block_tail():
    # 37 tokens x (5 + 1) rows is not a multiple of the 16 rows of a workgroup
    n = 37
    _run(1, n, 5, 64, [list(range(n))], BF16, seed=6)


def _full(wl):
    L = binding()
    inp = workloads.gen_prep(wl, seed=0)
    dt = wl.idx_dtype
    print(f"[full-size prep] {wl.name}", flush=True)
    q_out = torch.empty((wl.B, wl.n_q, wl.H, 128), dtype=TORCH[dt], device="cuda")
    k_cache = torch.zeros((wl.B, wl.n_kv, 128), dtype=TORCH[dt], device="cuda")
    lat_cache = torch.zeros((wl.B, wl.n_kv, wl.Dc), dtype=TORCH[wl.mla_dtype], device="cuda")
    L.dsa_indexer_prep(dev(inp["pos"]), q_in=dev(inp["q_in"]), q_out=q_out, k_in=dev(inp["k_in"]),
                       k_cache=k_cache, latent_in=dev(inp["latent_in"], wl.mla_dtype), latent_cache=lat_cache)
    torch.cuda.synchronize()
    qw, kw = oracle.indexer_prep(inp["q_in"], inp["k_in"], inp["pos"], 10000.0, dt, True)
    assert_storage_close(host(q_out.view(torch.int16)).view(np.uint16), qw, dt, f"{wl.name} q_out")
    pos = inp["pos"]
    bidx = np.repeat(np.arange(wl.B), wl.n_q)
    kg = host(k_cache.view(torch.int16)).view(np.uint16)[bidx, pos.reshape(-1)]
    assert_storage_close(kg, kw.reshape(-1, 128), dt, f"{wl.name} k rows")
    lg = host(lat_cache.view(torch.int16)).view(np.uint16)[bidx, pos.reshape(-1)]
    assert np.array_equal(lg, inp["latent_in"].reshape(-1, wl.Dc)), f"{wl.name} latent rows"


@pytest.mark.parametrize("name", ["batched_decode_b32_32k", "chunked_prefill_4096_after_12288",
                                  "long_decode_b8_128k", "glm_decode_b1_8k"])
def test_full_size(name):
    _full(workloads.WORKLOADS[name])
