"""The Python binding refuses caller-supplied tensors that a kernel would
read or write past (wrong size or dtype, other device, non-contiguous)
before anything is enqueued."""
import pytest
import torch

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402

DEV = torch.device("cuda:0")
CUBIC = [(1.5, -0.5, 0.0)]


def _x(r, c, dtype=torch.float32):
    return torch.randn(r, c, device=DEV).to(dtype)


def test_quantize_outputs_checked():
    x = _x(64, 128)
    with pytest.raises(ValueError):
        ns.nvfp4_quantize(x, codes=torch.empty(64, 32, dtype=torch.uint8, device=DEV))
    with pytest.raises(TypeError):
        ns.nvfp4_quantize(x, scales=torch.empty(64, 8, dtype=torch.int16, device=DEV))
    with pytest.raises(TypeError):
        ns.nvfp4_quantize(x, workspace=torch.empty(1024, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        ns.nvfp4_quantize(x.t())                          # not contiguous
    with pytest.raises(ValueError):
        ns.nvfp4_quantize_rht(x, 0x5A5A, global_scale=torch.empty(1, device="cpu"))


def test_dequantize_and_gemm_checked():
    x = _x(64, 256)
    q = ns.nvfp4_quantize(x)
    with pytest.raises(ValueError):
        ns.nvfp4_dequantize(*q, 64, 256, out=torch.empty(64, 128, device=DEV))
    with pytest.raises(ValueError):                       # codes too short for K = 512
        ns.nvfp4_gemm(q, q, 64, 64, 512, symmetric=True)
    with pytest.raises(ValueError):
        ns.nvfp4_gemm(q, q, 64, 64, 256, symmetric=True, out=torch.empty(64, 32, device=DEV))
    with pytest.raises(TypeError):
        ns.nvfp4_gemm(q, q, 64, 64, 256, symmetric=True,
                      amax_out=torch.zeros(1, dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        ns.nvfp4_gemm(q, q, 64, 64, 256, symmetric=True, beta=1.0,
                      addend=torch.empty(64, 32, device=DEV))


def test_ns_outputs_checked():
    G = _x(64, 128, torch.bfloat16)
    with pytest.raises(ValueError):
        ns.ns_orthogonalize(G, CUBIC, out=torch.empty(128, 64, device=DEV))
    with pytest.raises(TypeError):
        ns.ns_orthogonalize_ex(G, CUBIC, out=torch.empty(64, 128, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        ns.ns_abs_quantile(G, 0.99, out=torch.empty(0, device=DEV))
    Gs = [G, _x(32, 64, torch.bfloat16)]
    with pytest.raises(ValueError):                       # one output missing
        ns.ns_orthogonalize_grouped(Gs, CUBIC, [1.0, 1.0], outs=[torch.empty(64, 128, device=DEV)])
    with pytest.raises(ValueError):                       # second output of the wrong shape
        ns.ns_orthogonalize_grouped(Gs, CUBIC, [1.0, 1.0],
                                    outs=[torch.empty(64, 128, device=DEV),
                                          torch.empty(64, 32, device=DEV)])
    with pytest.raises(ValueError):
        ns.ns_orthogonalize_grouped(Gs, CUBIC, [1.0])      # one clip per matrix
