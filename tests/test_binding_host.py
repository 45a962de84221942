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
