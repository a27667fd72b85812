"""Calibration-driven block selection: block-replay SQNR and the policy rule ladder (oracle side).

The Quark Wan2.2 page ("Calibration-driven block selection") replays captured
BF16 block inputs through two quantized versions of each block, OFF (plain
dynamic MXFP4) and ON (MXFP4 behind a transform), computes the block output's
SQNR against the BF16 reference, and decides each block with a rule ladder
whose thresholds come in three tiers. Readings recorded in the design notes:

* SQNR = 10 log10( sum y_ref^2 / sum (y - y_ref)^2 ) in dB, over every output
  element of the block; a block here is its quantized linears (the path holds
  no attention or norms), each fed its captured input, and their outputs
  together form the block output. y is the quantized layer's output as the
  layer produces it, in bf16. No noise gives +inf, no signal -inf.
* The rules, first match wins, with best = max(sqnr_off, sqnr_on):
      best < floor                 -> bf16 (the block stays unquantized)
      best < w4a8_sqnr             -> W4A8
      sqnr_on - sqnr_off > margin  -> transform_on
      otherwise                    -> W4A4 (plain MXFP4)
  The comparisons are strict, as printed.
"""

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits
from .linear import EPI_NONE, W4A4, W4A8, TRANSFORM_ON, qdq_matmul
from .quant import mxfp4_quantize
from .transform import hadamard_channel_amax, mxfp4_quantize_hadamard, smoothquant_factors

BF16_MODE = 2

# tier -> (floor, w4a8_sqnr, margin) in dB, the page's tier table
TIERS = {
    "low": (8.0, 21.0, 0.5),
    "mid": (10.0, 23.0, 0.5),
    "high": (12.0, 25.0, 0.5),
}


def sqnr_sums(y, y_ref):
    """(sum y_ref^2, sum (y - y_ref)^2) in float64 over all elements."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    return float((r * r).sum()), float(((y - r) ** 2).sum())


def sqnr_db(signal, noise):
    """10 log10(signal / noise); +inf without noise, -inf without signal (0 / 0 counts as +inf)."""
    if noise == 0:
        return float("inf")
    if signal == 0:
        return float("-inf")
    return 10.0 * np.log10(signal / noise)


def select_mode(sqnr_off, sqnr_on, tier="high"):
    """One block's decision by the rule ladder."""
    floor, w4a8_sqnr, margin = TIERS[tier]
    best = max(sqnr_off, sqnr_on)
    if best < floor:
        return BF16_MODE
    if best < w4a8_sqnr:
        return W4A8
    if sqnr_on - sqnr_off > margin:
        return TRANSFORM_ON
    return W4A4


def select_policy(sqnr_off, sqnr_on, tier="high"):
    """[n_experts, n_blocks] SQNR tables -> uint8 policy artifact."""
    off = np.asarray(sqnr_off, dtype=np.float64)
    on = np.asarray(sqnr_on, dtype=np.float64)
    out = np.empty(off.shape, np.uint8)
    for idx in np.ndindex(off.shape):
        out[idx] = select_mode(float(off[idx]), float(on[idx]), tier)
    return out


def block_replay_sums(linears):
    """OFF and ON SQNR sums of one block.

    ``linears`` is a list of (x_bits [M, K], w_bits [N, K], y_ref [M, N]) with
    captured bf16 inputs, the linear's bf16 weight and its captured BF16 output.
    OFF quantizes x and W with plain MXFP4; ON calibrates the transform on the
    captured x and on W and quantizes both transformed. Returns
    ((signal, noise_off), (signal, noise_on))."""
    sig = n_off = n_on = 0.0
    for x, w, y_ref in linears:
        xc, xs = mxfp4_quantize(x)
        wc, ws = mxfp4_quantize(w)
        y_off = bf16_bits_to_f64(f64_to_bf16_bits(qdq_matmul(W4A4, xc, xs, wc, ws, None, EPI_NONE)))
        am, wm = smoothquant_factors(hadamard_channel_amax([x]), hadamard_channel_amax([w]))
        txc, txs = mxfp4_quantize_hadamard(x, am)
        twc, tws = mxfp4_quantize_hadamard(w, wm)
        y_on = bf16_bits_to_f64(f64_to_bf16_bits(qdq_matmul(W4A4, txc, txs, twc, tws, None, EPI_NONE)))
        s, e_off = sqnr_sums(y_off, y_ref)
        _, e_on = sqnr_sums(y_on, y_ref)
        sig += s
        n_off += e_off
        n_on += e_on
    return (sig, n_off), (sig, n_on)
