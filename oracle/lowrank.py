"""SVDQuant's low-rank branch beside the quantized linear (oracle side).

The Quark Wan2.2 page ("Mixed-Precision selection" and its note; "Results",
the SVDQuant rows) uses SVDQuant as a generation-time transform: activation
smoothing plus a low-rank correction kept in 16-bit beside the 4-bit product.
For a linear y = x W^T with W ~ L2^T L1^T + R (rank r, from an SVD computed
offline on trained weights) the layer is

    y = epilogue( Q(x) Q(R)^T + (x L1) L2 + bias )

with the residual R packed as MXFP4 like any weight and the branch run on the
unquantized bf16 activation. Readings recorded in the design notes (the pages
fix no arithmetic for the branch):

* The branch runs in bf16 like a pair of bf16 linears: T = RN_bf16(x L1), its
  sum exact here (fp32 accumulation on the GPU).
* The quantized product comes out of its GEMM as bf16 with the bias and
  without the GELU (y_pre); the branch is added to it, then the epilogue:
      y = RN_bf16( epilogue( y_pre + T L2 ) )
  with T L2 an exact sum here. GELU, when the linear has it, applies to the
  whole pre-activation.
* Layouts: L1 is given transposed, [r, K] (one rank vector per row, K
  contiguous), L2 as [N, r] (nn.Linear layout of the up projection).

A second reading runs the branch's second half inside the quantized product:
T L2 joins the quantized product's fp32 sums before the bias and the epilogue,
and the output is rounded to bf16 once (``svdquant_linear_fused``):

    y = RN_bf16( epilogue( Q(x) Q(R)^T + T L2 + bias ) )

with T = RN_bf16(x L1) as before. It differs from the first only by the bf16
rounding of y_pre that it leaves out.
"""

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits
from .linear import EPI_GELU_TANH, EPI_NONE, gelu_tanh, qdq_matmul


def lowrank_down(x_bits, l1t_bits):
    """T = RN_bf16(x L1) as bf16 bits [M, r], from x [M, K] and L1 transposed [r, K]."""
    x = bf16_bits_to_f64(np.asarray(x_bits, np.uint16))
    l1t = bf16_bits_to_f64(np.asarray(l1t_bits, np.uint16))
    return f64_to_bf16_bits(x @ l1t.T)


def lowrank_up(y_pre_bits, t_bits, l2_bits, epilogue=EPI_NONE):
    """y = RN_bf16(epilogue(y_pre + T L2^T')) as bf16 bits [M, N]; L2 in [N, r] layout."""
    y_pre = bf16_bits_to_f64(np.asarray(y_pre_bits, np.uint16))
    t = bf16_bits_to_f64(np.asarray(t_bits, np.uint16))
    l2 = bf16_bits_to_f64(np.asarray(l2_bits, np.uint16))
    v = y_pre + t @ l2.T
    if epilogue == EPI_GELU_TANH:
        v = gelu_tanh(v)
    elif epilogue != EPI_NONE:
        raise ValueError(f"unknown epilogue {epilogue}")
    return f64_to_bf16_bits(v)


def svdquant_linear_fused(mode, a_codes, a_scales, r_codes, r_scales, t_bits, l2_bits, bias=None,
                          epilogue=EPI_NONE):
    """float64 y [M, N] = epilogue(Q(x) Q(R)^T + T L2^T' + bias) before the output's bf16 rounding.

    T [M, r] is the branch's first half in bf16 bits (``lowrank_down``), L2 [N, r]."""
    t = bf16_bits_to_f64(np.asarray(t_bits, np.uint16))
    l2 = bf16_bits_to_f64(np.asarray(l2_bits, np.uint16))
    v = qdq_matmul(mode, a_codes, a_scales, r_codes, r_scales, None, EPI_NONE) + t @ l2.T
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64)[None, :]
    if epilogue == EPI_GELU_TANH:
        v = gelu_tanh(v)
    elif epilogue != EPI_NONE:
        raise ValueError(f"unknown epilogue {epilogue}")
    return v


def svdquant_linear(mode, a_codes, a_scales, r_codes, r_scales, x_bits, l1t_bits, l2_bits, bias=None,
                    epilogue=EPI_NONE):
    """The whole layer from the activation codes, the packed residual and the branch factors.

    Returns (y bf16 bits, y_pre bf16 bits, T bf16 bits)."""
    y_pre = f64_to_bf16_bits(qdq_matmul(mode, a_codes, a_scales, r_codes, r_scales, bias, EPI_NONE))
    t = lowrank_down(x_bits, l1t_bits)
    return lowrank_up(y_pre, t, l2_bits, epilogue), y_pre, t
