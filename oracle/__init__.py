"""Oracle for the NVFP4 Newton–Schulz path — TEST INFRASTRUCTURE ONLY.

A plain, slow, FP64 CPU implementation of what the GPU library computes,
written from "Full-Stack FP4: Stable LLM Pretraining with Quantized
Projections, Optimizers, and Attention" (arXiv 2607.04422):

* ``formats``  — the E2M1 element code and the FP8 E4M3 block-scale code of
  the NVFP4 format (§2 "Preliminaries", paragraph "NVFP4 format"), decoded by
  closed form and encoded by exact comparison (round to nearest, ties to even).
* ``nvfp4``    — the 1x16 / 16x1 block quantizer and the dequantizer
  (x_hat = x_E2M1 * s * s_g, §2 "NVFP4 format"; RTN per §3.4).
* ``rht``      — the random 16 x 16 Hadamard transform that §3.4 applies to
  every quantized operand along the contraction axis.
* ``quantile`` — the p99 clip threshold as an order statistic of |G| (§3.4
  p99 outlier clipping, App. F Table 8 quantile ratio 0.99).
* ``native``   — a ctypes loader of the C++ oracle (``cpp/nvfp4_oracle.cpp``): a
  second, independently written quantizer and float64 NVFP4 NS loop with
  OpenMP, pinned like this package and cross-checked against it; the
  benchmark times it on the host cores.
* ``ns``       — the Newton–Schulz iteration of the Root optimizer, exact
  (§2 "Root optimizer") and with NVFP4 operands (§3.4, the three-line NVFP4
  NS iteration, with or without the transform), plus the caller-side clip
  and Frobenius normalisation.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.

Pins (what each function is checked against, in ``tests/test_oracle_*.py``):
codecs against the format's closed form and torch's float8_e4m3fn cast;
rounding against brute-force nearest-grid search with exact rationals;
round-trip of exactly representable tensors; idempotence; the per-block error
bound; the FP64 GEMM against a pure-Python triple loop; the Hadamard matrix
against its recursive construction, its orthogonality, the transform against
its definition in plain loops, the FP32 butterfly against the FP64 product,
and the cancellation of the transform in every NS product; adaptive 4/6
block choices against a brute-force rebuild of both candidates over every
scale byte and code; the quantile against sorting and the library's
inverted-CDF quantile; exact NS against the
SVD closed form of its scalar map and, for the cubic, the polar factor; the
quantized NS against the scalar map on matrices whose quantization is benign.
The quantized NS on general inputs has no pin beyond the composition of these
(its end-to-end values are not printed anywhere): parity unpinned for that
composition on general inputs.
"""
from .formats import (E2M1_MAGNITUDES, e2m1_decode, e4m3fn_decode,
                      e4m3fn_encode_quotient, e2m1_encode_quotient)
from .nvfp4 import (tensor_amax, global_scale, quantize_rows, quantize_cols,
                    dequantize_rows, dequantize_cols, round_to_bf16,
                    NVFP4Tensor)
from .ns import (clip_and_normalize, gemm_nt, ns_exact, ns_nvfp4, ns_nvfp4_step,
                 ns_iteration_flops)

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_decode", "e4m3fn_decode",
    "e4m3fn_encode_quotient", "e2m1_encode_quotient",
    "tensor_amax", "global_scale", "quantize_rows", "quantize_cols",
    "dequantize_rows", "dequantize_cols", "round_to_bf16", "NVFP4Tensor",
    "clip_and_normalize", "gemm_nt", "ns_exact", "ns_nvfp4", "ns_nvfp4_step",
    "ns_iteration_flops",
]
