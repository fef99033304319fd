"""Argument checks of the Python binding (no GPU needed). The C ABI takes raw
addresses and cannot see a tensor's dtype, size or device, so the binding
rejects misuse before calling the library: wrong integer widths for
seq_lens / block_table / dst_rows, wrong output dtypes, sizes that do not
match the shape, non-contiguous tensors and host tensors."""
import numpy as np
import pytest
import torch

import kv_cache_vector_rotation_amd as tq


def test_dtype_checked_before_use():
    with pytest.raises(ValueError, match="dtype"):
        tq._dev(torch.zeros(3, dtype=torch.int64), "seq_lens", torch.int32)   # [1000, 517, 33] as int64
    with pytest.raises(ValueError, match="dtype"):
        tq._dev(torch.zeros(4, dtype=torch.int32), "dst_rows", torch.int64)
    with pytest.raises(ValueError, match="dtype"):
        tq._dev(torch.zeros(4, dtype=torch.float64), "out", torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        tq._dev(torch.zeros((2, 3), dtype=torch.int64), "block_table", torch.int32)


def test_size_and_layout_checked():
    with pytest.raises(ValueError, match="elements"):
        tq._dev(torch.zeros(5, dtype=torch.float32), "out", torch.float32, numel=6)
    with pytest.raises(ValueError, match="at least"):
        tq._dev(torch.zeros(5, dtype=torch.int32), "cache.codes", torch.int32, min_numel=6)
    with pytest.raises(ValueError, match="contiguous"):
        tq._dev(torch.zeros((4, 4), dtype=torch.float32).t(), "q", torch.float32)


def test_host_tensor_rejected():
    # a host address handed to a kernel would fault the GPU
    with pytest.raises(ValueError, match="GPU"):
        tq._dev(torch.zeros(4, dtype=torch.float32), "logits", torch.float32, numel=4)
    with pytest.raises(ValueError, match="GPU"):
        tq._call_device(torch.zeros(4), "q")


def test_missing_required_and_optional():
    with pytest.raises(ValueError, match="required"):
        tq._dev(None, "out", torch.float32)
    assert tq._dev(None, "logits", torch.float32, optional=True) is None


def test_entry_points_reject_host_inputs():
    rng = np.random.default_rng(0)
    rot = np.linalg.qr(rng.standard_normal((128, 128)))[0]
    sk = rng.standard_normal((128, 128)).astype(np.float32)
    kq = tq.Quantizer.from_parts([rot], [sk], [2], device="cpu")
    kc = tq.Cache.empty(kq, 64, tq.TQ_TOKEN_MAJOR, device="cpu")
    vc = tq.Cache.empty(kq, 64, tq.TQ_BLOCK32, device="cpu")
    shape = tq.decode_shape(1, 4, 1, 64, 64, 0.1)
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    out = torch.zeros((1, 4, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_attn_decode(kq, kq, shape, q, kc, vc, out=out)
    with pytest.raises(ValueError, match="GPU"):
        tq.tq_attn_decode_scratch(kq, kq, shape, q, kc, vc, out=out)
    with pytest.raises(ValueError):
        tq.tq_quantize(kq, tq.TQ_TOKEN_MAJOR, torch.zeros((8, 128)), kc)
    with pytest.raises(ValueError):
        tq.tq_search(kq, kc, 64, torch.zeros((3, 128)), 10)
