"""Seeded synthetic inputs for the MX quantized linear workloads.

This module only draws inputs: it holds none of the quantization or GEMM
arithmetic, and both the oracle-side tests and the GPU-side tests/benchmark
take their inputs from here.

Recipe (shapes from the Wan2.2 workloads; the pages ship no weights, prompts or
activations, so these seeded draws stand in for them):

* Host draws use ``numpy.random.default_rng([config_id, expert, block, tensor_id])``.
* Activations X [M, K]: standard normal float32; then outlier channels
  (columns along K): either ``k`` seeded columns multiplied by a factor
  ("scaled" kind), or round(0.005 K) seeded columns replaced by 10 * Student-t
  (nu = 3) samples ("student_t" kind, the heavy-tailed outlier channels that
  motivate W4A8 on the pages). Then a round-to-nearest-even cast to bf16.
* Weights W [N, K] (nn.Linear order, K contiguous): normal with std 0.02,
  drawn directly in [N, K] order, cast to bf16.
* Large weight stacks (dozens of blocks of 5120-wide linears) are drawn on the
  GPU with torch's seeded Philox generator instead, so that a whole stack can
  be produced in seconds; a test that checks such a weight copies the drawn
  bf16 tensor back to the host and hands it to the oracle.
* Policy masks: ``rng.choice(n_blocks, k, replace=False)`` per expert; two
  experts whose draws coincide are redrawn.

bf16 values on the host are uint16 bit patterns.
"""

from dataclasses import dataclass, field

import numpy as np

W4A4 = 0
W4A8 = 1

# tensor_id values used when seeding
T_X_VIDEO = 0
T_X_TEXT = 1
T_MASK = 2
T_WEIGHT_BASE = 100  # + linear index within a block


def rng(config_id, expert=0, block=0, tensor_id=0):
    return np.random.default_rng([int(config_id), int(expert), int(block), int(tensor_id)])


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even (torch cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def n_student_t_outliers(k):
    return int(round(0.005 * k))


def activation_bf16(config_id, m, k, outliers, expert=0, block=0, tensor_id=T_X_VIDEO):
    """X [m, k] bf16 bits. ``outliers`` is ("scaled", n_cols, factor), ("student_t",) or None."""
    g = rng(config_id, expert, block, tensor_id)
    x = g.standard_normal((m, k), dtype=np.float32)
    if outliers is not None and k > 0:
        kind = outliers[0]
        if kind == "scaled":
            _, n_cols, factor = outliers
            cols = g.choice(k, size=n_cols, replace=False)
            x[:, cols] *= np.float32(factor)
        elif kind == "student_t":
            n_cols = n_student_t_outliers(k)
            cols = g.choice(k, size=n_cols, replace=False)
            x[:, cols] = (10.0 * g.standard_t(3, size=(m, n_cols))).astype(np.float32)
        else:
            raise ValueError(kind)
    return f32_to_bf16_bits(x)


def weight_bf16(config_id, n, k, expert=0, block=0, linear=0):
    """W [n, k] bf16 bits, normal with std 0.02."""
    g = rng(config_id, expert, block, T_WEIGHT_BASE + linear)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return f32_to_bf16_bits(w)


def weight_bf16_device(config_id, n, k, expert=0, block=0, linear=0, device="cuda"):
    """W [n, k] bf16 torch tensor drawn on the device (seeded Philox), std 0.02."""
    import torch

    seed = (((int(config_id) * 7919 + int(expert)) * 1009 + int(block)) * 131 + int(linear)) & ((1 << 63) - 1)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w = torch.randn((n, k), generator=gen, device=device, dtype=torch.float32)
    w.mul_(0.02)
    return w.to(torch.bfloat16)


def policy_mask(config_id, n_experts, n_blocks, n_w4a8):
    """uint8 [n_experts, n_blocks] table: n_w4a8 seeded W4A8 blocks per expert, rest W4A4."""
    table = np.full((n_experts, n_blocks), W4A4, dtype=np.uint8)
    chosen = []
    for e in range(n_experts):
        attempt = 0
        while True:
            g = rng(config_id, e, attempt, T_MASK)
            pick = tuple(sorted(int(i) for i in g.choice(n_blocks, size=n_w4a8, replace=False)))
            if pick not in chosen or n_w4a8 in (0, n_blocks):
                break
            attempt += 1
        chosen.append(pick)
        table[e, list(pick)] = W4A8
    return table


@dataclass(frozen=True)
class Linear:
    name: str
    m_role: str  # "video" or "text" (which activation feeds it) or "ffn_hidden"
    k: int
    n: int
    epilogue: int = 0  # 0 none, 1 tanh-GELU


@dataclass
class Workload:
    config_id: int
    name: str
    m_video: int
    m_text: int
    dim: int
    ffn: int
    n_experts: int
    n_blocks: int
    n_w4a8: int  # per expert; -1 means "all blocks use fixed_mode"
    fixed_mode: int = W4A4
    linears: tuple = field(default_factory=tuple)
    outliers: tuple = ("student_t",)
    explicit_policy: tuple = ()

    def policy(self):
        if self.explicit_policy:
            return np.array(self.explicit_policy, dtype=np.uint8)
        if self.n_w4a8 < 0:
            return np.full((self.n_experts, self.n_blocks), self.fixed_mode, dtype=np.uint8)
        return policy_mask(self.config_id, self.n_experts, self.n_blocks, self.n_w4a8)

    def m_of(self, lin):
        return self.m_text if lin.m_role == "text" else self.m_video

    def flops_per_block(self):
        return sum(2 * self.m_of(l) * l.n * l.k for l in self.linears)

    def total_flops(self):
        return self.flops_per_block() * self.n_blocks * self.n_experts


def _ffn(dim, ffn):
    return (Linear("ffn_up", "video", dim, ffn, 1), Linear("ffn_down", "ffn_hidden", ffn, dim, 0))


def _a14b_block(dim=5120, ffn=13824):
    return (
        Linear("self_q", "video", dim, dim),
        Linear("self_k", "video", dim, dim),
        Linear("self_v", "video", dim, dim),
        Linear("self_o", "video", dim, dim),
        Linear("cross_q", "video", dim, dim),
        Linear("cross_k", "text", dim, dim),
        Linear("cross_v", "text", dim, dim),
        Linear("cross_o", "video", dim, dim),
    ) + _ffn(dim, ffn)


def _ti2v_block(dim=3072, ffn=14336):
    return (
        Linear("self_q", "video", dim, dim),
        Linear("self_k", "video", dim, dim),
        Linear("self_v", "video", dim, dim),
        Linear("self_o", "video", dim, dim),
    ) + _ffn(dim, ffn) + (
        Linear("cross_k", "text", dim, dim),
        Linear("cross_v", "text", dim, dim),
    )


def workload(config_id):
    """The five synthetic workloads, by id (1 = tiny ... 5 = full A14B 720p stack)."""
    if config_id == 1:
        # one linear, run once per mode: block 0 is W4A4, block 1 is W4A8
        return Workload(1, "tiny_qlinear_256x512x512", 256, 0, 512, 0, 1, 2, -1, W4A4,
                        (Linear("tiny", "video", 512, 512),), ("scaled", 4, 20.0),
                        ((W4A4, W4A8),))
    if config_id == 2:
        return Workload(2, "a14b_self_attn_qkv_480p_w4a4", 32760, 0, 5120, 0, 1, 1, -1, W4A4,
                        (Linear("qkv", "video", 5120, 15360),))
    if config_id == 3:
        return Workload(3, "a14b_ffn_720p_w4a8", 75600, 0, 5120, 13824, 1, 1, -1, W4A8,
                        _ffn(5120, 13824))
    if config_id == 4:
        return Workload(4, "ti2v5b_30block_mixed", 11440, 512, 3072, 14336, 1, 30, 5, W4A4,
                        _ti2v_block())
    if config_id == 5:
        return Workload(5, "a14b_40block_2expert_720p_mixed", 75600, 512, 5120, 13824, 2, 40, 6, W4A4,
                        _a14b_block())
    raise ValueError(config_id)
