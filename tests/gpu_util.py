"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
arrays, and oracle comparisons on full or sampled rows."""

import contextlib
import os

import numpy as np
import torch

import oracle


def dev_bf16(bits):
    """uint16 bf16 bits (host) -> bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def host_bits(t):
    """bf16 tensor -> uint16 bits on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.detach().cpu().numpy().view(np.uint8)


def host_f32(t):
    return t.detach().cpu().numpy().astype(np.float32)


def group_major_scales(scales_rows):
    """[rows, K/32] E8M0 bytes (oracle order) -> [ceil(K/128), rows, 4] (library order), zero padded."""
    s = np.asarray(scales_rows, np.uint8)
    rows, kb = s.shape
    g = (kb + 3) // 4
    pad = np.zeros((rows, 4 * g), np.uint8)
    pad[:, :kb] = s
    return np.ascontiguousarray(pad.reshape(rows, g, 4).transpose(1, 0, 2))


def panel_index(n_rows, K, bits, rows=None):
    """Byte indices of K-panel-major codes, as [len(rows), K * bits / 8] in row-major order.

    The library stores codes in panels of 128 elements along K (the last one
    narrower when K % 128 != 0); panel p holds every row's codes of its range,
    row after row. This is the documented permutation the tests undo before
    comparing with the oracle's row-major codes.
    """
    rows = np.arange(n_rows, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    full = 128 * bits // 8
    parts = []
    for p in range((K + 127) // 128):
        w = min(128, K - 128 * p) * bits // 8
        parts.append(p * full * n_rows + rows[:, None] * w + np.arange(w, dtype=np.int64)[None, :])
    return np.concatenate(parts, axis=1)


def code_rows(codes, n_rows, K, bits, rows=None):
    """Host row-major codes [len(rows), K * bits / 8] of a device K-panel-major code buffer."""
    idx = panel_index(n_rows, K, bits, rows)
    flat = codes.reshape(-1)
    got = flat[torch.from_numpy(idx.reshape(-1)).to(flat.device)]
    return got.cpu().numpy().view(np.uint8).reshape(idx.shape)


def sample_rows(m, n_sample, seed, tile=256):
    """Seeded row sample that always holds row 0, row m-1 and rows of the last tile."""
    g = np.random.default_rng(seed)
    last = np.arange(max(0, (m - 1) // tile * tile), m)
    pick = g.choice(m, size=min(n_sample, m), replace=False)
    rows = np.unique(np.concatenate([[0, m - 1], last[-8:], pick]))
    return rows.astype(np.int64)


def assert_codes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: " \
                          f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}"


def assert_output_close(y_bits, y_ref, what):
    y = oracle.bf16_bits_to_f64(y_bits)
    rep = oracle.output_error_report(y, y_ref)
    assert rep["finite"], f"{what}: non-finite output"
    assert rep["worst_ratio"] <= 1.0, f"{what}: tolerance exceeded {rep}"
    return rep


# The pipelined W4A4 GEMM has a four-wave and an eight-wave kernel; the
# library picks one by the launch's size, and MXQ_W4A4_WAVES (read at every
# call) fixes the choice so that either one can be tested on any shape.
W4A4_WAVE_KERNEL = {4: "pipe_w4a4_wg256x256_wave128x128", 8: "pipe_w4a4_wg256x256_wave128x64"}


@contextlib.contextmanager
def w4a4_waves(waves):
    old = os.environ.get("MXQ_W4A4_WAVES")
    os.environ["MXQ_W4A4_WAVES"] = str(waves)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MXQ_W4A4_WAVES", None)
        else:
            os.environ["MXQ_W4A4_WAVES"] = old
