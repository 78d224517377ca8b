"""The Python binding refuses caller-supplied buffers whose shape, dtype,
device or layout the kernels would not fit (the C ABI takes plain pointers
and cannot check sizes), before any launch."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_forward_and_backward_buffers():
    q = _t(1, 100, 2, 64)
    with pytest.raises(ValueError):
        fa.forward(q, q, q, lse=_t(1, 2, 99, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.forward(q, q, q, out=_t(1, 100, 2, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.forward(q, q, q, out=_t(1, 100, 2, 128)[..., :64])  # not contiguous
    o, lse = fa.forward(q, q, q)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, o, q, lse[:, :, :50])
    with pytest.raises(ValueError):
        fa.backward(q, q, q, o, q, lse, workspace=_t(1, 2, 100, dtype=torch.float16))
    with pytest.raises(ValueError):
        fa.backward(q, q, q, o, q, lse, dq=_t(1, 100, 2, 32))
    with pytest.raises(ValueError):
        fa.backward_dkdv(q, q, q, q, lse, _t(2, 100, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.backward_dq(q, q, q, q, lse.cpu(), _t(1, 2, 100, dtype=torch.float32))
    torch.cuda.synchronize()


def test_variant_buffers():
    q = _t(1, 256, 2, 128)
    with pytest.raises(ValueError):
        fa.quantize_fp8(q, 128, scales=_t(1, 2, 1, dtype=torch.float32))
    q8, qs = fa.quantize_fp8(q, 128)
    k8, ks = fa.quantize_fp8(q, 64)
    with pytest.raises(ValueError):
        fa.forward_fp8_quantized(q8, k8, q, ks, ks)  # q scales have one entry per 128 rows
    with pytest.raises(ValueError):
        fa.forward_splitkv(q[:, :1].contiguous(), q, q, True, 4,
                           workspace=_t(10, dtype=torch.float32))
    cu = torch.tensor([0, 100, 256], dtype=torch.int32, device="cuda")
    p = q[0].contiguous()
    with pytest.raises(ValueError):
        fa.forward_varlen(p, p, p, cu, 156, lse=_t(2, 255, dtype=torch.float32))
    torch.cuda.synchronize()
