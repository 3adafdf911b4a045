"""The Python binding checks every buffer before it calls the library (CPU only).

The C ABI receives raw pointers, so a wrong dtype, shape, stride, device, format,
layout or size of a caller's buffer can only be caught in the binding.  These tests
swap the library for a wrapper that answers the host-only size queries from the real
library and fails the test if any compute entry point is reached, then check that each
bad argument raises ValueError first.  Tensors live on the CPU here (the binding's
device check is lifted for the test; on a GPU every buffer must be a CUDA tensor of
one device).
"""
import pytest
import torch

from activation_sparsity_fp4_sharq_amd import sharq

HOST_ONLY = {"sharq_abi_version", "sharq_status_str", "sharq_payload_bytes", "sharq_prep_workspace_bytes",
             "sharq_linear_workspace_bytes", "sharq_prep_rmsnorm_workspace_bytes"}


class _NoComputeLib:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in HOST_ONLY:
            return getattr(self._real, name)

        def reached(*args, **kwargs):
            raise AssertionError(f"{name} was called although an argument is invalid")
        return reached


@pytest.fixture
def stub(monkeypatch):
    monkeypatch.setattr(sharq, "_lib", _NoComputeLib(sharq.lib()))
    monkeypatch.setattr(sharq, "_REQUIRE_CUDA", False)
    monkeypatch.setattr(sharq, "_stream", lambda stream=None: None)


def payload(rows, K, fmt=sharq.MXFP4, layout=None):
    return sharq.Payload.empty(rows, K, fmt, torch.device("cpu"), layout)


def test_host_payload_sizes_match_the_library():
    for rows, K, fmt, layout in [(1, 32, 0, 0), (37, 96, 0, 1), (300, 1056, 0, 1), (5, 64, 1, 0), (0, 64, 0, 1)]:
        assert sharq._host_payload_sizes(rows, K, fmt, layout) == sharq.payload_sizes(rows, K, fmt, layout)


def test_library_abi_version_matches_the_binding():
    assert sharq.lib().sharq_abi_version() == sharq.ABI_VERSION


def test_linear_output_dtype_must_match(stub):
    bb, rr, w = payload(64, 128), payload(64, 128), payload(32, 128)
    y = torch.empty((64, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        sharq.linear(bb, rr, w, sharq.OUT_FP32, y=y)  # fp32 stores into a bf16 buffer would overrun it


@pytest.mark.parametrize("shape", [(64, 31), (63, 32), (64, 33), (32, 64)])
def test_linear_output_shape_must_match(stub, shape):
    bb, rr, w = payload(64, 128), payload(64, 128), payload(32, 128)
    with pytest.raises(ValueError, match="shape"):
        sharq.linear(bb, rr, w, sharq.OUT_BF16, y=torch.empty(shape, dtype=torch.bfloat16))


def test_linear_output_needs_unit_column_stride(stub):
    bb, rr, w = payload(64, 128), payload(64, 128), payload(32, 128)
    y = torch.empty((32, 64), dtype=torch.bfloat16).t()
    with pytest.raises(ValueError, match="stride"):
        sharq.linear(bb, rr, w, sharq.OUT_BF16, y=y)


def test_linear_payloads_must_agree(stub):
    w = payload(32, 128)
    with pytest.raises(ValueError, match="expected"):
        sharq.linear(payload(64, 256), payload(64, 256), w)  # K differs from the weight's
    with pytest.raises(ValueError, match=r"\[64"):
        sharq.linear(payload(64, 128), payload(65, 128), w)  # residual rows differ
    with pytest.raises(ValueError, match="format"):
        sharq.linear(payload(64, 128, sharq.NVFP4), payload(64, 128, sharq.NVFP4), w)
    with pytest.raises(ValueError, match="layout"):
        sharq.linear(payload(64, 128, layout=sharq.ROWMAJOR), payload(64, 128, layout=sharq.ROWMAJOR), w)


def test_payload_buffers_must_be_large_enough(stub):
    bb, rr, w = payload(64, 128), payload(64, 128), payload(32, 128)
    short = sharq.Payload(bb.codes[:-16], bb.scales, bb.tensor_scale, bb.fmt, bb.layout, 64, 128)
    with pytest.raises(ValueError, match="needs"):
        sharq.linear(short, rr, w)
    wrong = sharq.Payload(bb.codes.view(torch.int8), bb.scales, bb.tensor_scale, bb.fmt, bb.layout, 64, 128)
    with pytest.raises(ValueError, match="uint8"):
        sharq.linear(wrong, rr, w)


def test_tiled_nvfp4_is_rejected(stub):
    bad = sharq.Payload(torch.empty(4096, dtype=torch.uint8), torch.empty(512, dtype=torch.uint8),
                        torch.ones(4), sharq.NVFP4, sharq.TILED, 32, 128)
    with pytest.raises(ValueError, match="layout"):
        sharq.linear(bad, bad, payload(32, 128, sharq.NVFP4))


def test_prep_outputs_are_checked(stub):
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="expected"):
        sharq.prep(x, out=(payload(64, 256), payload(64, 256)))
    with pytest.raises(ValueError, match="share a layout"):
        sharq.prep(x, out=(payload(64, 128, layout=sharq.TILED), payload(64, 128, layout=sharq.ROWMAJOR)))
    with pytest.raises(ValueError, match="workspace"):
        sharq.prep(x, fmt=sharq.NVFP4, out=(payload(64, 128, sharq.NVFP4), payload(64, 128, sharq.NVFP4)),
                   ws=torch.empty(8, dtype=torch.uint8))


def test_prep_input_is_checked(stub):
    with pytest.raises(ValueError, match="bfloat16"):
        sharq.prep(torch.zeros((64, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        sharq.prep(torch.zeros((128, 64), dtype=torch.bfloat16).t())


def test_forward_checks_every_buffer(stub):
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    w = payload(32, 128)
    with pytest.raises(ValueError, match="dtype"):
        sharq.forward(x, w, out_dtype=sharq.OUT_FP32, y=torch.empty((64, 32), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="expected"):
        sharq.forward(x, payload(32, 256))
    with pytest.raises(ValueError, match="expected"):
        sharq.bind_forward(x, w, bufs=(payload(64, 128), payload(60, 128)))


def test_dequantize_output_is_checked(stub):
    p = payload(8, 64)
    with pytest.raises(ValueError, match="dtype"):
        sharq.dequantize(p, out=torch.empty((8, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        sharq.dequantize(p, out=torch.empty((8, 32), dtype=torch.float32))


def test_cuda_is_required_outside_these_tests():
    with pytest.raises(ValueError, match="CUDA"):
        sharq.prep(torch.zeros((4, 64), dtype=torch.bfloat16))
