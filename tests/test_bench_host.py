"""Host-side logic of bench.py and of the synthetic workloads it times (CPU only).

The workload sizes are restated from the configurations they stand for (token
counts from the latent grids, Wan2.2 A14B and TI2V-5B widths), so a wrong
dimension or a dropped linear in the workload table changes a FLOP count here.
"""

import hashlib
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_token_counts_follow_the_latent_grids():
    assert synth.workload(2).m_video == 21 * 30 * 52
    assert synth.workload(3).m_video == 21 * 45 * 80
    assert synth.workload(4).m_video == 13 * 22 * 40
    assert synth.workload(5).m_video == 21 * 45 * 80
    assert synth.workload(4).m_text == synth.workload(5).m_text == 512


def test_flops_per_step_of_each_workload():
    assert synth.workload(1).total_flops() == 2 * (2 * 256 * 512 * 512)  # once per mode
    assert synth.workload(2).total_flops() == 2 * 32760 * 5120 * 15360
    assert synth.workload(3).total_flops() == 2 * (2 * 75600 * 5120 * 13824)
    ti2v_block = 4 * 2 * 11440 * 3072 ** 2 + 2 * 2 * 11440 * 3072 * 14336 + 2 * 2 * 512 * 3072 ** 2
    assert synth.workload(4).total_flops() == 30 * ti2v_block
    a14b_block = (6 * 2 * 75600 * 5120 ** 2 + 2 * 2 * 512 * 5120 ** 2 + 2 * 2 * 75600 * 5120 * 13824)
    assert synth.workload(5).total_flops() == 2 * 40 * a14b_block


def test_policy_masks_match_the_mixed_configurations():
    p4 = synth.workload(4).policy()
    assert p4.shape == (1, 30) and int((p4 == synth.W4A8).sum()) == 5
    assert set(np.unique(p4)) <= {synth.W4A4, synth.W4A8}
    p5 = synth.workload(5).policy()
    assert p5.shape == (2, 40)
    assert all(int((p5[e] == synth.W4A8).sum()) == 6 for e in range(2))
    assert not np.array_equal(p5[0], p5[1])  # each expert has its own mask
    assert np.array_equal(p5, synth.workload(5).policy())  # seeded: the same every call
    assert np.all(synth.workload(3).policy() == synth.W4A8)
    assert np.all(synth.workload(2).policy() == synth.W4A4)


def _write_summary(root, tag, sha, rows):
    os.makedirs(os.path.join(root, "profiles"))
    os.makedirs(os.path.join(root, "mx_bit_quantized_amd", "csrc"))
    with open(os.path.join(root, "mx_bit_quantized_amd", "csrc", "mxq_gemm.hip"), "wb") as f:
        f.write(b"// kernel source stand-in\n")
    with open(os.path.join(root, "profiles", f"hbm_traffic_{tag}.txt"), "w") as f:
        f.write("# header\n")
        f.write(f"source_sha1_gemm {sha}\n")
        for r in rows:
            f.write(" ".join(str(x) for x in r) + "\n")


def test_profiled_traffic_weights_instances_by_dispatches(tmp_path, monkeypatch):
    sha = hashlib.sha1(b"// kernel source stand-in\n").hexdigest()
    _write_summary(str(tmp_path), "w", sha, [
        ("kernel", "gemm_pipe_kernel<0,128,4,false,false,false,false>", 3, 0, 0, 1000),
        ("kernel", "gemm_pipe_kernel<0,128,4,true,false,true,false>", 1, 0, 0, 5000),
        ("kernel", "gemm_pipe_kernel<1,128,3,false,false,false,false>", 2, 0, 0, 700),
        ("kernel", "mxfp4_quant_kernel", 9, 0, 0, 123),
    ])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("w", 0) == (3 * 1000 + 5000) // 4
    assert bench.profiled_traffic("w", 1) == 700
    assert bench.profiled_traffic("missing", 0) is None


def test_profiled_traffic_is_null_once_the_kernel_source_changes(tmp_path, monkeypatch):
    _write_summary(str(tmp_path), "w", "0" * 40, [
        ("kernel", "gemm_pipe_kernel<0,128,4,false,false,false,false>", 3, 0, 0, 1000)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("w", 0) is None


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_fused_projections_cover_every_linear_once_with_the_same_flops():
    """exec_linears stacks only linears that read one input, keeps K, role and epilogue, and does not
    change the work: each linear in exactly one GEMM, the GEMMs' FLOPs summing to the workload's."""
    for cfg in (1, 2, 3, 4, 5):
        wl = synth.workload(cfg)
        for fuse in (False, True):
            ex = bench.exec_linears(wl.linears, fuse)
            parts = [p for _, p in ex]
            assert sorted(i for p in parts for i in p) == list(range(len(wl.linears)))
            flops = sum(2 * wl.m_of(lin) * lin.n * lin.k for lin, _ in ex)
            assert flops * wl.n_experts * wl.n_blocks == wl.total_flops()
            for lin, p in ex:
                members = [wl.linears[i] for i in p]
                assert lin.n == sum(m.n for m in members)
                assert all((m.k, m.m_role, m.epilogue) == (lin.k, lin.m_role, lin.epilogue) for m in members)
                assert len({bench.input_group(m.name) for m in members}) == 1
            if not fuse:
                assert all(len(p) == 1 for p in parts)
    five = [lin.name for lin, _ in bench.exec_linears(synth.workload(5).linears, True)]
    assert five == ["self_q+self_k+self_v", "self_o", "cross_q", "cross_k+cross_v", "cross_o", "ffn_up", "ffn_down"]


def test_fused_projection_that_does_not_fit_stays_split():
    wl = synth.workload(5)
    ex = bench.exec_linears(wl.linears, True, fits=lambda lin: lin.n * wl.m_of(lin) * 2 < 2 ** 31)
    names = [lin.name for lin, _ in ex]
    assert names[:3] == ["self_q", "self_k", "self_v"] and "cross_k+cross_v" in names
    assert sorted(i for _, p in ex for i in p) == list(range(len(wl.linears)))
