"""The Python binding fails loudly instead of computing anywhere else: a missing library is
an ImportError, and host (CPU) tensors are refused before any call into the library. No GPU
is touched."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_attention_10_amd import dsa  # noqa: E402


def test_missing_library_is_an_import_error(monkeypatch, tmp_path):
    monkeypatch.setattr(dsa, "LIB_PATH", str(tmp_path / "libdsa.so"))
    with pytest.raises(ImportError, match="missing"):
        dsa._load()


def _cpu(*shape, dtype=torch.float32):
    return torch.zeros(*shape, dtype=dtype)


def test_index_score_refuses_host_tensors():
    q, k = _cpu(1, 1, 4, 128, dtype=torch.bfloat16), _cpu(1, 64, 128, dtype=torch.bfloat16)
    w, s = _cpu(1, 1, 4), _cpu(1, 1, 64)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.dsa_index_score(q, k, w, s)


def test_topk_refuses_host_tensors():
    with pytest.raises(ValueError, match="device tensor"):
        dsa.dsa_topk(_cpu(2, 64), _cpu(2, 8, dtype=torch.int32), 8)


def test_sparse_mla_refuses_host_tensors():
    qa, lat = _cpu(1, 1, 16, 576, dtype=torch.bfloat16), _cpu(1, 64, 576, dtype=torch.bfloat16)
    idx, out = _cpu(1, 1, 16, dtype=torch.int32), _cpu(1, 1, 16, 512)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.dsa_sparse_mla_attn(qa, lat, idx, out, 512, 0.0625)


class _NoLib:
    """Stands in for libdsa: any call into it fails the test (validation must refuse first)."""
    def __getattr__(self, name):
        def call(*a, **k):
            raise AssertionError(f"{name} called although the arguments are invalid")
        return call


@pytest.fixture
def host_binding(monkeypatch):
    """The binding's checks on host tensors: device placement is taken as given, and the
    library must never be reached."""
    monkeypatch.setattr(dsa, "_dev", lambda t, n: None)
    monkeypatch.setattr(dsa, "lib", _NoLib())
    return dsa


def test_sparse_mla_checks_lse_and_kv_len(host_binding):
    d = host_binding
    qa, lat = _cpu(2, 1, 16, 576, dtype=torch.bfloat16), _cpu(2, 64, 576, dtype=torch.bfloat16)
    idx, out = _cpu(2, 1, 16, dtype=torch.int32), _cpu(2, 1, 16, 512)
    for lse in (_cpu(2, 1, 8), _cpu(2, 16), _cpu(2, 1, 16, dtype=torch.float16)):
        with pytest.raises(ValueError, match="lse"):
            d.dsa_sparse_mla_attn(qa, lat, idx, out, 512, 0.0625, lse=lse)
    for kv in (_cpu(2, dtype=torch.int64), _cpu(3, dtype=torch.int32), _cpu(2, 1, dtype=torch.int32)):
        with pytest.raises(ValueError, match="kv_len"):
            d.dsa_sparse_mla_attn(qa, lat, idx, out, 512, 0.0625, kv_len=kv)


def test_index_score_checks_kv_len_and_q_pos(host_binding):
    d = host_binding
    q, k = _cpu(2, 3, 4, 128, dtype=torch.bfloat16), _cpu(2, 64, 128, dtype=torch.bfloat16)
    w, s = _cpu(2, 3, 4), _cpu(2, 3, 64)
    for kv in (_cpu(2, dtype=torch.int64), _cpu(1, dtype=torch.int32)):
        with pytest.raises(ValueError, match="kv_len"):
            d.dsa_index_score(q, k, w, s, kv_len=kv)
    for qp in (_cpu(2, 3, dtype=torch.int64), _cpu(2, dtype=torch.int32), _cpu(2, 4, dtype=torch.int32)):
        with pytest.raises(ValueError, match="q_pos"):
            d.dsa_index_score(q, k, w, s, q_pos=qp)


def test_kpool_calls_check_lse_kv_len_q_pos(host_binding):
    d = host_binding
    qa, lat = _cpu(2, 1, 16, 512, dtype=torch.bfloat16), _cpu(2, 64, 512, dtype=torch.bfloat16)
    pidx, packed = _cpu(2, 1, 4, dtype=torch.int32), _cpu(2, 64, 257, dtype=torch.float16)
    out = _cpu(2, 1, 16, 512)
    with pytest.raises(ValueError, match="lse"):
        d.dsa_kpool_sparse_mla_attn(qa, lat, pidx, packed, 128, 4, out, 512, 0.0625, lse=_cpu(2, 1, 15))
    with pytest.raises(ValueError, match="q_pos"):
        d.dsa_kpool_sparse_mla_attn(qa, lat, pidx, packed, 128, 4, out, 512, 0.0625,
                                    q_pos=_cpu(2, 1, dtype=torch.int64))
    tok = _cpu(2, 1, 19, dtype=torch.int32)
    with pytest.raises(ValueError, match="kv_len"):
        d.dsa_kpool_expand(pidx, packed, 128, tok, 4, kv_len=_cpu(2, dtype=torch.int64))
