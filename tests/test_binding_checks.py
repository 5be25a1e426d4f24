"""The Python binding rejects host tensors, wrong element types and short
buffers before anything reaches the library (CPU: the checks raise before
any pointer is used)."""
import pytest
import torch

import block_mean_pool_amd as sa


class FakeDevice:
    """Stands in for a device tensor: what the binding's checks read."""

    def __init__(self, dtype, numel, offset=0):
        self.is_cuda = True
        self.device = "cuda:0"
        self.dtype = dtype
        self._numel = numel
        self._offset = offset
        self._esize = torch.empty((), dtype=dtype).element_size()

    def element_size(self):
        return self._esize

    def storage_offset(self):
        return self._offset

    def numel(self):
        return self._numel

    def untyped_storage(self):
        nbytes = (self._numel + self._offset) * self._esize

        class S:
            def nbytes(self_inner):
                return nbytes
        return S()

    def data_ptr(self):  # pragma: no cover - never reached by these tests
        raise AssertionError("pointer used although the check should have raised")


P = sa.make_params(1, 2, 300, 128, dtype="bf16")
N_QKV = 2 * 300 * 128


def test_host_tensor_rejected():
    q = torch.zeros(1, 2, 300, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        sa.sparse_attn_predict(P, q, q, sa.SaMask(), None)


def test_wrong_dtype_rejected():
    q = FakeDevice(torch.float32, N_QKV)
    with pytest.raises(TypeError, match="bfloat16"):
        sa.sparse_attn_predict(P, q, q, sa.SaMask(), None)


def test_short_buffer_rejected():
    q = FakeDevice(torch.bfloat16, N_QKV - 1)
    with pytest.raises(ValueError, match="elements"):
        sa.sparse_attn_predict(P, q, q, sa.SaMask(), None)
    # a view that starts inside its storage has that much less room
    q = FakeDevice(torch.bfloat16, N_QKV, offset=0)
    k = FakeDevice(torch.bfloat16, N_QKV - 64, offset=64)
    with pytest.raises(ValueError, match="elements"):
        sa.sparse_attn_predict(P, q, k, sa.SaMask(), None)


def test_strided_extent():
    # [B, N, H, D] storage described by strides: N rows of H * D elements
    p = sa.make_params(1, 2, 300, 128, dtype="bf16", strides=(0, 128, 256))
    assert sa._extent(p) == 299 * 256 + 128 + 128
    q = FakeDevice(torch.bfloat16, 299 * 256 + 255)
    with pytest.raises(ValueError, match="elements"):
        sa.sparse_attn_predict(p, q, q, sa.SaMask(), None)


def test_outputs_checked():
    q = FakeDevice(torch.bfloat16, N_QKV)
    o_bad = FakeDevice(torch.float32, N_QKV)
    with pytest.raises(TypeError, match="bfloat16"):
        sa.sparse_attn_forward(P, q, q, q, sa.SaMask(), o_bad)
    p32 = sa.make_params(1, 2, 300, 128, dtype="bf16", o_fp32=True)
    lse_short = FakeDevice(torch.float32, 2 * 300 - 1)
    with pytest.raises(ValueError, match="lse"):
        sa.sparse_attn_forward(p32, q, q, q, sa.SaMask(), o_bad, lse_short)
    skip_bad = FakeDevice(torch.float32, 10**6)
    with pytest.raises(TypeError, match="skip_bits"):
        sa.sparse_attn_forward(p32, q, q, q, sa.SaMask(), o_bad, None, skip_bad)


def test_mask_and_reorder_buffers_checked():
    with pytest.raises(TypeError, match="kept_idx"):
        sa.make_mask(FakeDevice(torch.int64, 10), FakeDevice(torch.int32, 10))
    with pytest.raises(ValueError, match="device tensor"):
        sa.make_reorder(torch.zeros(10, dtype=torch.int32), FakeDevice(torch.int32, 10))


def test_permute_checks_element_size():
    x = FakeDevice(torch.float32, N_QKV)
    y = FakeDevice(torch.bfloat16, N_QKV)
    perm = FakeDevice(torch.int32, 600)
    with pytest.raises(TypeError, match="4-byte|2-byte"):
        sa.sparse_attn_permute(P, x, perm, 0, y)
