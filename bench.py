"""Benchmark of the MX quantized linear hot path on one MI355X.

A step is one forward pass of every quantized linear of the workload (the
policy lookup, activation quantization and scaled GEMM of each linear, the
FFN's GELU epilogue and the re-quantization of its hidden state), with all
inputs and packed weights already resident in HBM. Linears that read the same
tensor in the model (self-attention q, k, v; cross-attention k, v) share one
quantization of it and run as one GEMM over their weights stacked along N, the
usual fused projection (--separate-qkv runs one GEMM each on the shared
codes; the outputs are the same column for column). Weight packing is offline
and is timed separately (reported, not part of the step).

    python bench.py [--steps K] [--warmup W] [--workload a14b_stack|a14b_ffn|qkv|ti2v|tiny]
                    [--act-scale per_token|static] [--transform-on] [--svdquant-rank R] [--select]
                    [--token-shards S] [--separate-qkv]

--act-scale static runs the W4A8 linears on static (per-tensor) FP8
activations: each input's amax is calibrated once, untimed, on the same
synthetic inputs, and the FFN's first projection of a W4A8 block writes the
hidden state's static FP8 codes itself. The default is the per-token scale.

--transform-on runs every W4A4 block as transform_on: block Hadamard rotation
plus SmoothQuant ahead of MXFP4. The factors are calibrated once, untimed, on
the same synthetic inputs and on each weight, and the weights are packed
transformed. Such a block's FFN first projection rotates, rescales and
quantizes the hidden state for the second one in its epilogue
(mxq_gemm_mxfp4_hadamard_out), as the plain W4A4 FFN does without the
transform.

--svdquant-rank R adds SVDQuant's rank-R bf16 branch to every W4A4 linear:
T = x L1 (in the quantizer's pass over x where the linear quantizes its own
input), then the GEMM on the residual with T L2 in its fp32 sums and the
epilogue (one kernel; shapes the pipelined GEMM does not take run the GEMM
without epilogue, then y = epilogue(y_pre + T L2)). The FFN's first
projection writes its bf16 hidden state, which the second one's branch reads.
A fused projection (q+k+v, cross-attention k+v) is one linear there too, with
one branch whose L2 spans its stacked columns (--separate-qkv gives each of
its linears a branch of its own). The factors are random bf16 of the right
shapes (no trained weights to decompose); the branch's cost does not depend
on their values.

--select replaces the step by the calibration-driven block selection over the
A14B model (see run_select).

--token-shards S times one GPU's share of the workload split S ways along the
video tokens (ceil(M / S) rows; text rows and all weights whole on every GPU),
the exchange-free split of this path. The line reports that one GPU's rate.

Prints one JSON line. Per-launch kernel durations come from HIP events
recorded on the launch stream around every kernel of the last timed step (the
other timed steps run without them: the events cost 1.4% of a full-size step).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "W4A4/W4A8 qlinear TFLOP/s + % MFMA peak at Wan2.2-A14B 720p shapes"
PEAK_TFLOPS = {0: 10100.0, 1: 5000.0}  # dense MFMA: fp4 (W4A4), fp8 (W4A8 issues at the fp8 rate)
PEAK_HBM_GBS = 8000.0
WORKLOADS = {"tiny": 1, "qkv": 2, "a14b_ffn": 3, "ti2v": 4, "a14b_stack": 5}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="a14b_stack", choices=sorted(WORKLOADS))
    ap.add_argument("--act-scale", default="per_token", choices=["per_token", "static"],
                    help="W4A8 activation scale: per token (amax/448 of each row) or static per tensor (calibrated)")
    ap.add_argument("--transform-on", action="store_true",
                    help="run the W4A4 blocks as transform_on (Hadamard rotation + SmoothQuant, calibrated)")
    ap.add_argument("--svdquant-rank", type=int, default=0, choices=[0, 32, 64, 96, 128],
                    help="add SVDQuant's low-rank bf16 branch of this rank to every W4A4 linear")
    ap.add_argument("--select", action="store_true",
                    help="instead of the step: calibration-driven block selection over the A14B model (one 480p "
                         "calibration sample), timing the library's block replay")
    ap.add_argument("--token-shards", type=int, default=1,
                    help="time one GPU's share of the workload split over this many GPUs along the video tokens "
                         "(M / S rows each; text rows and weights whole on every GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true", help="leave out roofline.measured_peak")
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (calibrates HBM byte counters) and exit")
    ap.add_argument("--peak", action="store_true",
                    help="only measure the roofline denominators: the register-only scaled-MFMA rate (FP4xFP4, "
                         "FP4xFP8) on random operands and a device copy, with clock and socket power, and exit")
    ap.add_argument("--gemm-power", action="store_true",
                    help="only run the A14B W4A4 GEMM (75600 x 5120 x 5120, both wave counts) and the A14B W4A8 "
                         "FFN GEMMs (up with GELU, down) back to back, on random and on constant data, sampling "
                         "socket power and clock, and exit")
    ap.add_argument("--separate-qkv", action="store_true",
                    help="run q, k, v (and cross-attention k, v) as separate GEMMs on their shared quantized input "
                         "instead of one GEMM over the stacked weights")
    ap.add_argument("--peak-seconds", type=float, default=1.0,
                    help="seconds per MFMA probe (the default bench line runs them for this long too)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class PowerSampler:
    """Socket power and gfx clock, sampled with amd-smi in a thread while a region runs.

    The board holds a power cap by lowering the clock, so these say whether a
    measured rate was capped. Reports medians (None where amd-smi is absent)."""

    def __init__(self, period=0.5):
        import threading
        self.period, self.samples, self._stop = period, [], threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import subprocess
        while not self._stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                d = json.loads(r.stdout)
                d = d[0] if isinstance(d, list) else d
                d = d["gpu_data"][0] if "gpu_data" in d else d
                val = lambda v: v.get("value") if isinstance(v, dict) else v
                pw = val(d.get("power", {}).get("socket_power"))
                ck = val((d.get("clock", {}).get("gfx_0") or {}).get("clk"))
                if isinstance(pw, (int, float)) and isinstance(ck, (int, float)):
                    self.samples.append((float(pw), float(ck)))
            except Exception:
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        if not self.samples:
            return {"socket_w": None, "gfx_mhz": None, "samples": 0}
        # the first sample can predate the load
        body = self.samples[1:] if len(self.samples) > 2 else self.samples
        return {"socket_w": float(np.median([p for p, _ in body])), "gfx_mhz": float(np.median([c for _, c in body])),
                "samples": len(body)}


def gemm_power(torch, mxq, seconds=4.0):
    """The A14B W4A4 GEMM, then the A14B W4A8 FFN GEMMs, each run back to back
    for `seconds` per case, with socket power and clock.

    Cases: the four- and eight-wave W4A4 kernels (MXQ_W4A4_WAVES) and the W4A8
    FFN up (GELU) and down projections, on random activations and weights (the
    synthetic distribution) and on constant ones.
    Shows whether the kernel's rate is set by its schedule or by the board's
    power cap: a capped kernel holds the cap and drops its clock."""
    dev = "cuda:0"
    m, n, k = 75600, 5120, 5120
    out = []
    for data in ("random", "constant"):
        if data == "random":
            g = torch.Generator(device=dev).manual_seed(3)
            x = torch.randn((m, k), generator=g, device=dev).to(torch.bfloat16)
            w = (torch.randn((n, k), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        else:
            x = torch.full((m, k), 1.5, device=dev).to(torch.bfloat16)
            w = torch.full((n, k), 0.03, device=dev).to(torch.bfloat16)
        wc, ws = mxq.quantize_weight_mxfp4(w)
        ac, asc = mxq.quantize_act(mxq.W4A4, x)
        del x, w
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        for waves in (4, 8):
            os.environ["MXQ_W4A4_WAVES"] = str(waves)
            for _ in range(5):
                mxq.gemm(mxq.W4A4, ac, asc, wc, ws, y=y)
            torch.cuda.synchronize()
            launches = 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with PowerSampler() as ps:
                t0 = time.time()
                e0.record()
                while time.time() - t0 < seconds:
                    for _ in range(10):
                        mxq.gemm(mxq.W4A4, ac, asc, wc, ws, y=y)
                    launches += 10
                    torch.cuda.synchronize()
                e1.record()
                torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / launches
            out.append({"data": data, "kernel": mxq.gemm_kernel_name(mxq.W4A4, m, n, k), "avg_us": round(us, 1),
                        "tflops": round(2 * m * n * k / us / 1e6, 1), **ps.summary()})
            log(json.dumps(out[-1]))
        os.environ.pop("MXQ_W4A4_WAVES", None)
        del ac, asc, wc, ws, y
        torch.cuda.empty_cache()
    # W4A8: the A14B FFN's two projections (per-token FP8 activations), same protocol
    for name, (m8, n8, k8, epi) in (("ffn_up_gelu", (75600, 13824, 5120, mxq.EPI_GELU_TANH)),
                                    ("ffn_down", (75600, 5120, 13824, mxq.EPI_NONE))):
        for data in ("random", "constant"):
            if data == "random":
                g = torch.Generator(device=dev).manual_seed(5)
                x = torch.randn((m8, k8), generator=g, device=dev).to(torch.bfloat16)
                w = (torch.randn((n8, k8), generator=g, device=dev) * 0.02).to(torch.bfloat16)
            else:
                x = torch.full((m8, k8), 1.5, device=dev).to(torch.bfloat16)
                w = torch.full((n8, k8), 0.03, device=dev).to(torch.bfloat16)
            wc, ws = mxq.quantize_weight_mxfp4(w)
            ac, asc = mxq.quantize_act(mxq.W4A8, x)
            del x, w
            y = torch.empty((m8, n8), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, epi, y)
            torch.cuda.synchronize()
            launches = 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with PowerSampler() as ps:
                t0 = time.time()
                e0.record()
                while time.time() - t0 < seconds:
                    for _ in range(4):
                        mxq.gemm(mxq.W4A8, ac, asc, wc, ws, None, epi, y)
                    launches += 4
                    torch.cuda.synchronize()
                e1.record()
                torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / launches
            out.append({"data": data, "linear": name, "kernel": mxq.gemm_kernel_name(mxq.W4A8, m8, n8, k8),
                        "avg_us": round(us, 1), "tflops": round(2 * m8 * n8 * k8 / us / 1e6, 1), **ps.summary()})
            log(json.dumps(out[-1]))
            del ac, asc, wc, ws, y
            torch.cuda.empty_cache()
    return out


def measure_peaks(torch, seconds):
    """Roofline denominators measured on this GPU (mxq_probe.hip).

    mfma: the register-only scaled MFMA of the GEMMs on random operands, one
    wave per SIMD on every CU, FP4 x FP4 (W4A4) and FP4 x FP8 (W4A8), each run
    for about `seconds`, with the shader clock of the run and the board's
    socket power; copy: a device copy of 2 GiB (read + write bytes)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "mx_bit_quantized_amd", "libmxq_probe.so"))
    lib.mxq_probe_mfma_words.restype = ctypes.c_size_t
    lib.mxq_probe_mfma_words.argtypes = [ctypes.c_int]
    lib.mxq_probe_mfma.restype = ctypes.c_int
    lib.mxq_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.mxq_probe_copy.restype = ctypes.c_int
    lib.mxq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    dev = "cuda:0"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus  # one 4-wave workgroup per CU: one wave per SIMD
    words = lib.mxq_probe_mfma_words(grid)
    g = torch.Generator(device=dev).manual_seed(77)
    rnd = torch.randint(-2 ** 31, 2 ** 31 - 1, (words * 4,), dtype=torch.int32, device=dev, generator=g)
    out = torch.empty((grid * 256,), dtype=torch.float32, device=dev)
    clk = torch.zeros((1,), dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    res = {}
    for name, fp8, flops_per_mfma in (("fp4xfp4", 0, 2 * 32 * 32 * 64), ("fp4xfp8", 1, 2 * 32 * 32 * 64)):
        def run(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert lib.mxq_probe_mfma(fp8, grid, iters, P(rnd), P(out), P(clk), stream) == 0
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3
        t = run(256)
        iters = max(256, int(256 * seconds / 4 / max(t, 1e-6)))  # about seconds / 4 per launch
        run(iters)  # warm the clock and power state
        with PowerSampler() as ps:
            ts, cycles = [], []
            for _ in range(4):
                ts.append(run(iters))
                cycles.append(int(clk.item()))
        flops = grid * 4 * iters * 128 * flops_per_mfma
        best = min(ts)
        res[name] = {"tflops": round(flops / best / 1e12, 1), "clock_ghz": round(cycles[ts.index(best)] / best / 1e9, 3),
                     **ps.summary()}
    del rnd, out
    n = (2 << 30) // 16
    src = torch.ones((n * 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        assert lib.mxq_probe_copy(P(src), P(dst), n, cus * 8, stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        assert lib.mxq_probe_copy(P(src), P(dst), n, cus * 8, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    res["copy_gbs"] = round(5 * 2 * n * 16 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return res


# Linears that read the same tensor in the model: self-attention q, k and v
# take the same normalized hidden state, cross-attention k and v the same text
# context. Their activation codes are computed once (by the first of them) and
# feed each GEMM; every other linear quantizes its own input, also where the
# synthetic data repeat a tensor.
SHARED_INPUT = {"self_k": "self_q", "self_v": "self_q", "cross_v": "cross_k"}


def input_group(name):
    """The first linear reading the same input as `name` (itself if none)."""
    return SHARED_INPUT.get(name, name)


def exec_linears(linears, fuse, fits=lambda lin: True):
    """The GEMMs of one block, as (Linear, [indices into `linears`]).

    With `fuse`, the linears that read one input (SHARED_INPUT: q, k, v;
    cross-attention k, v) run as one GEMM over their weights stacked along N,
    the usual fused projection: every output column is computed as by its own
    GEMM (same codes, same K order), and one launch replaces three or two.
    A stacked GEMM for which `fits` is false stays split into its linears."""
    out = []
    lead = {}
    for li, lin in enumerate(linears):
        g = input_group(lin.name)
        if fuse and g != lin.name and g in lead:
            i = lead[g]
            l0, parts = out[i]
            out[i] = (synth.Linear(l0.name + "+" + lin.name, l0.m_role, l0.k, l0.n + lin.n, l0.epilogue), parts + [li])
        else:
            lead[lin.name] = len(out)
            out.append((lin, [li]))
    split = []
    for lin, parts in out:
        split += [(lin, parts)] if len(parts) == 1 or fits(lin) else [(linears[i], [i]) for i in parts]
    return split


class Stack:
    """Packed weights, inputs and buffers of one workload on the device."""

    def __init__(self, wl, torch, mxq, static=False, transform=False, lr_rank=0, fuse=True):
        self.wl, self.torch, self.mxq = wl, torch, mxq
        # the GEMMs of a block: fused projections where the pipelined kernel takes
        # the stacked shape in both modes (every Wan2.2 shape here, A14B's 720p
        # q+k+v with its 2.3 GB output included). With SVDQuant a fused
        # projection is one linear with one branch of the given rank, as any
        # other linear (its factors are those of the stacked weight)
        pipelined = lambda lin: all(mxq.gemm_kernel_name(md, wl.m_of(lin), lin.n, lin.k).startswith("pipe_")
                                    for md in (0, 1))
        ex = exec_linears(wl.linears, fuse, pipelined)
        self.lins = [l for l, _ in ex]
        self.parts = [p for _, p in ex]
        self.static = static
        self.transform = transform
        self.lr_rank = lr_rank
        dev = "cuda:0"
        t0 = time.time()
        self.policy_table = wl.policy()
        self.policy = mxq.Policy(self.policy_table)
        self.li_down = next((i for i, l in enumerate(self.lins) if l.name == "ffn_down"), None)
        to_dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
        self.x_video = to_dev(synth.activation_bf16(wl.config_id, wl.m_video, wl.dim, wl.outliers,
                                                    tensor_id=synth.T_X_VIDEO))
        self.x_text = None
        if wl.m_text:
            self.x_text = to_dev(synth.activation_bf16(wl.config_id, wl.m_text, wl.dim, wl.outliers,
                                                       tensor_id=synth.T_X_TEXT))
        log(f"activations ready in {time.time() - t0:.1f}s")
        m_max = wl.m_video
        n_max = max(l.n for l in self.lins)
        self.y = torch.empty((m_max * n_max,), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((wl.m_video * max(wl.ffn, 1),), dtype=torch.bfloat16, device=dev)
        ws = max(mxq.qlinear_workspace_bytes(md, m_max, l.k) for md in (0, 1) for l in wl.linears)
        self.codes_buf = torch.empty((ws,), dtype=torch.uint8, device=dev)
        # W4A4 FFN: the first projection writes the second one's MXFP4 input here
        self.codes_buf2 = torch.empty((ws,), dtype=torch.uint8, device=dev)
        # transform_on: rotated per-channel maxima of the shared inputs, and each
        # linear's activation factors
        self.act_mult = {}
        # Linears that read one input share its factors, as SmoothQuant folds the
        # activation factor into the op that produces that input: lambda comes
        # from the input's maxima and the largest of their weights' maxima (so
        # q, k, v, and cross k, v, keep sharing one quantized input).
        self.aw_group = {}
        if transform:
            self.ax_role = {"video": mxq.hadamard_channel_amax(self.x_video)}
            if self.x_text is not None:
                self.ax_role["text"] = mxq.hadamard_channel_amax(self.x_text)
            grouped = {input_group(n) for n in SHARED_INPUT}
            for e in range(wl.n_experts):
                for b in range(wl.n_blocks):
                    if self.policy.mode(e, b) != 0:
                        continue
                    for li, lin in enumerate(self.lins):
                        g = input_group(lin.name)
                        if g in grouped:
                            w = self._weight(e, b, li)
                            self.aw_group[(e, b, g)] = mxq.hadamard_channel_amax(w, self.aw_group.get((e, b, g)))
                            del w
        # packed weights: drawn on the device per linear, packed, bf16 copy freed
        self.weights = {}
        pack_bytes, pack_ms = 0, 0.0
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for e in range(wl.n_experts):
            for b in range(wl.n_blocks):
                for li, lin in enumerate(self.lins):
                    w = self._weight(e, b, li)
                    codes = torch.empty((lin.n, lin.k // 2), dtype=torch.uint8, device=dev)
                    scales = torch.empty(mxq.mx_scale_shape(lin.n, lin.k), dtype=torch.uint8, device=dev)
                    tr = transform and self.policy.mode(e, b) == 0
                    if tr:
                        # calibration (untimed): the input's and the weight's rotated
                        # maxima give the factors; the weight is packed transformed
                        aw = self.aw_group.get((e, b, input_group(lin.name)))
                        if aw is None:
                            aw = mxq.hadamard_channel_amax(w)
                        ax = ax_h if lin.m_role == "ffn_hidden" else self.ax_role[lin.m_role]
                        am, wm = mxq.smoothquant_factors(ax, aw)
                        self.act_mult[(e, b, li)] = am
                    ev0.record()
                    if tr:
                        mxq.quantize_mxfp4_hadamard(w, wm, codes, scales)
                    else:
                        mxq.quantize_weight_mxfp4(w, codes, scales)
                    ev1.record()
                    torch.cuda.synchronize()
                    if tr and lin.name == "ffn_up":
                        # the hidden state of this block, for the second projection's maxima
                        m = wl.m_of(lin)
                        ac, asc = self._act_views(0, m, lin.k)
                        xin = self.x_video if lin.m_role == "video" else self.x_text
                        mxq.quantize_mxfp4_hadamard(xin, am, ac, asc)
                        hv = self.h[: m * lin.n].view(m, lin.n)
                        mxq.gemm(0, ac, asc, codes, scales, None, lin.epilogue, hv)
                        ax_h = mxq.hadamard_channel_amax(hv)
                    pack_ms += ev0.elapsed_time(ev1)
                    pack_bytes += lin.n * lin.k * 2 + lin.n * lin.k // 2 + lin.n * lin.k // 32
                    self.weights[(e, b, li)] = (codes, scales)
                    del w
        self.pack_gbs = pack_bytes / (pack_ms * 1e-3) / 1e9
        log(f"weights packed in {time.time() - t0:.1f}s ({pack_bytes / 1e9:.1f} GB traffic, {self.pack_gbs:.0f} GB/s)")
        # SVDQuant branch factors of the W4A4 linears (random bf16, seeded) and T's buffer
        self.lowrank = {}
        if lr_rank:
            gen = torch.Generator(device=dev).manual_seed(1234)
            for e in range(wl.n_experts):
                for b in range(wl.n_blocks):
                    if self.policy.mode(e, b) != 0:
                        continue
                    for li, lin in enumerate(self.lins):
                        l1t = (torch.randn((lr_rank, lin.k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
                        l2 = (torch.randn((lin.n, lr_rank), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
                        self.lowrank[(e, b, li)] = (l1t, l2)
            self.t_buf = torch.empty((m_max * lr_rank,), dtype=torch.bfloat16, device=dev)
        self.records = []  # (kind, mode, flops, bytes, ev_start, ev_end)
        self.down_ready = False  # the FFN's second projection has its input codes in codes_buf2
        if static:
            self._calibrate()

    def _weight(self, e, b, i):
        """bf16 weight of GEMM i of block (e, b): its linears' synthetic weights stacked along N."""
        wl = self.wl
        ws = [synth.weight_bf16_device(wl.config_id, wl.linears[p].n, wl.linears[p].k, e, b, p) for p in self.parts[i]]
        return ws[0] if len(ws) == 1 else self.torch.cat(ws, dim=0)

    def _calibrate(self):
        """Static FP8 scales (untimed): the amax of each W4A8 input tensor over the synthetic inputs.

        Video and text activations are shared by every linear that reads them;
        the FFN hidden state of each W4A8 block is calibrated on the output of
        its first projection, run once on static activations."""
        torch, mxq, wl = self.torch, self.mxq, self.wl
        t0 = time.time()
        self.amax = {"video": mxq.fp8_calibrate(self.x_video)}
        if self.x_text is not None:
            self.amax["text"] = mxq.fp8_calibrate(self.x_text)
        self.amax_h = {}
        for e in range(wl.n_experts):
            for b in range(wl.n_blocks):
                if self.policy.mode(e, b) != 1:
                    continue
                for li, lin in enumerate(self.lins):
                    if lin.name != "ffn_up":
                        continue
                    m = wl.m_of(lin)
                    codes, scales = self._act_views(1, m, lin.k)
                    mxq.quantize_act_fp8_static(self.x_video if lin.m_role == "video" else self.x_text,
                                                self.amax[lin.m_role], codes, scales)
                    h = self.h[: m * lin.n].view(m, lin.n)
                    wc, wsc = self.weights[(e, b, li)]
                    mxq.gemm(1, codes, scales, wc, wsc, None, lin.epilogue, h)
                    self.amax_h[(e, b)] = mxq.fp8_calibrate(h)
        torch.cuda.synchronize()
        log(f"static FP8 scales calibrated in {time.time() - t0:.1f}s ({len(self.amax_h)} FFN hidden states)")

    def _input_amax(self, e, b, role):
        return self.amax_h[(e, b)] if role == "ffn_hidden" else self.amax[role]

    def _act_views(self, mode, m, k, buf=None):
        torch = self.torch
        buf = self.codes_buf if buf is None else buf
        if mode == 0:
            cb = m * k // 2
            codes = buf[:cb].view(m, k // 2)
            off = (cb + 255) // 256 * 256
            shape = self.mxq.mx_scale_shape(m, k)
            scales = buf[off:off + shape[0] * m * 4].view(shape)
        else:
            cb = m * k
            codes = buf[:cb].view(m, k)
            off = (cb + 255) // 256 * 256
            scales = buf[off:off + 4 * m].view(torch.float32)
        return codes, scales

    def step(self, timed):
        torch, mxq, wl = self.torch, self.mxq, self.wl
        for e in range(wl.n_experts):
            for b in range(wl.n_blocks):
                mode = self.policy.mode(e, b)
                codes_src = None  # the linear whose activation codes codes_buf holds
                for li, lin in enumerate(self.lins):
                    m = wl.m_of(lin)
                    if lin.m_role == "video":
                        x = self.x_video
                    elif lin.m_role == "text":
                        x = self.x_text
                    else:
                        x = self.h[: m * lin.k].view(m, lin.k)
                    out = (self.h if lin.epilogue == 1 else self.y)[: m * lin.n].view(m, lin.n)
                    wc, wsc = self.weights[(e, b, li)]
                    # FFN: the first projection quantizes its GELU output for
                    # the second one in its epilogue (same codes as quantizing
                    # its bf16 output), the second one reads them as they are.
                    # W4A4: MXFP4 (transform_on: rotated and rescaled by the
                    # second projection's factors first); W4A8: only with static
                    # scales (a per-token scale needs the row's amax first)
                    static8 = mode == 1 and self.static
                    tr = mode == 0 and self.transform
                    lr = self.lowrank.get((e, b, li)) if mode == 0 else None
                    # SVDQuant: the branch's second half runs inside the GEMM where the
                    # pipelined kernel takes the shape; the FFN's second projection needs
                    # the bf16 hidden state for its own branch, so the first one keeps it
                    lr_fused = lr is not None and mxq.gemm_lowrank_supported(m, lin.n, lin.k)
                    fused_up = lin.name == "ffn_up" and lr is None and (
                        (mode == 0 and mxq.gemm_mxfp4_out_supported(m, lin.n, lin.k))
                        or (static8 and mxq.gemm_fp8_static_out_supported(m, lin.n, lin.k)))
                    fed = lin.name == "ffn_down" and self.down_ready
                    # (transform_on: the linears of one input share its factors too)
                    shared = codes_src is not None and SHARED_INPUT.get(lin.name) == codes_src
                    if fed:
                        codes, scales = self._act_views(mode, m, lin.k, self.codes_buf2)
                    else:
                        codes, scales = self._act_views(mode, m, lin.k)
                    if timed:
                        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                        e0.record()
                    # a branch linear that quantizes its own input takes T in the same pass over x
                    quant_lr = lr is not None and not fed and not shared
                    if lr is not None:
                        t = self.t_buf[: m * self.lr_rank].view(m, self.lr_rank)
                    if quant_lr:
                        codes_src = lin.name
                        mxq.quantize_act_lowrank(x, lr[0], codes, scales, t)
                    elif not fed and not shared:
                        codes_src = lin.name
                        if tr:
                            mxq.quantize_mxfp4_hadamard(x, self.act_mult[(e, b, li)], codes, scales)
                        elif static8:
                            mxq.quantize_act_fp8_static(x, self._input_amax(e, b, lin.m_role), codes, scales)
                        else:
                            mxq.quantize_act(mode, x, codes, scales)
                    if timed:
                        e1.record()
                    if lr is not None and not quant_lr:
                        mxq.lowrank_down(x, lr[0], t)
                    if timed:
                        e1b = torch.cuda.Event(enable_timing=True)
                        e1b.record()
                    if lr_fused:
                        mxq.gemm_lowrank(codes, scales, wc, wsc, t, lr[1], None, lin.epilogue, y=out)
                        out_bytes = m * lin.n * 2 + (m + lin.n) * self.lr_rank * 2
                    elif fused_up and tr:
                        # the second projection's rotation and factors, in the epilogue
                        oc, osc = self._act_views(mode, m, lin.n, self.codes_buf2)
                        mxq.gemm_mxfp4_hadamard_out(codes, scales, wc, wsc, self.act_mult[(e, b, self.li_down)],
                                                    None, lin.epilogue, oc, osc)
                        out_bytes = m * lin.n // 2 + m * lin.n // 32
                    elif fused_up and mode == 0:
                        oc, osc = self._act_views(mode, m, lin.n, self.codes_buf2)
                        mxq.gemm_mxfp4_out(codes, scales, wc, wsc, None, lin.epilogue, oc, osc)
                        out_bytes = m * lin.n // 2 + m * lin.n // 32
                    elif fused_up:
                        oc, osc = self._act_views(mode, m, lin.n, self.codes_buf2)
                        mxq.gemm_fp8_static_out(codes, scales, wc, wsc, self.amax_h[(e, b)], None, lin.epilogue,
                                                oc, osc)
                        out_bytes = m * lin.n + 4 * m
                    elif lr is not None:
                        # the quantized product without the epilogue, then the branch and the epilogue
                        mxq.gemm(mode, codes, scales, wc, wsc, None, 0, out)
                        out_bytes = m * lin.n * 2
                    else:
                        mxq.gemm(mode, codes, scales, wc, wsc, None, lin.epilogue, out)
                        out_bytes = m * lin.n * 2
                    if timed:
                        e2.record()
                    if lr is not None and not lr_fused:
                        mxq.lowrank_up(out, t, lr[1], lin.epilogue, y=out)
                    self.down_ready = fused_up
                    if timed:
                        e5 = torch.cuda.Event(enable_timing=True)
                        e5.record()
                        qbytes = m * lin.k * 2 + (m * lin.k // 2 + m * lin.k // 32 if mode == 0 else m * lin.k + 4 * m)
                        gbytes = ((m * lin.k // 2 + m * lin.k // 32) if mode == 0 else (m * lin.k + 4 * m)) \
                            + lin.n * lin.k // 2 + lin.n * lin.k // 32 + out_bytes
                        if quant_lr:
                            self.records.append(("quant_lowrank", mode, 2 * m * self.lr_rank * lin.k,
                                                 qbytes + m * self.lr_rank * 2, e0, e1))
                        elif not fed and not shared:
                            self.records.append(("quant", mode, 0, qbytes, e0, e1))
                        # the GEMM's flops are those of the quantized product (the branch's
                        # 2 m n r bf16 flops inside the fused kernel are not counted)
                        self.records.append(("gemm", mode, 2 * m * lin.n * lin.k, gbytes, e1b, e2))
                        if lr is not None and not quant_lr:
                            rr = self.lr_rank
                            self.records.append(("lowrank_down", mode, 2 * m * rr * lin.k,
                                                 m * lin.k * 2 + m * rr * 2, e1, e1b))
                            if not lr_fused:
                                self.records.append(("lowrank_up", mode, 2 * m * rr * lin.n,
                                                     2 * m * lin.n * 2, e2, e5))


# the pipelined GEMM's symbol per mode, as the profile summaries write it
# (template arguments: mode, K elements per stage, ring depth, GELU, bias,
# MXFP4 output; no spaces): each mode has several instances, and the
# roofline covers all of them
KERNEL_SYMBOL = {0: "gemm_pipe_kernel<0,128,4,*>", 1: "gemm_pipe_kernel<1,128,3,*>"}
KERNEL_PREFIX = {0: "gemm_pipe_kernel<0,128,4,", 1: "gemm_pipe_kernel<1,128,3,"}


def profiled_traffic(workload_tag, mode):
    """HBM bytes per launch of the mode's GEMM kernels from the committed counter summary.

    profiles/hbm_traffic_<workload>.txt holds calibrated FETCH_SIZE + WRITE_SIZE
    bytes per dispatch and the sha1 of the GEMM source they were taken on; a
    different source means the numbers describe another kernel: None. The
    instances of a mode are averaged, weighted by their dispatch counts.
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_tag}.txt")
    src = os.path.join(ROOT, "mx_bit_quantized_amd", "csrc", "mxq_gemm.hip")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha1(open(src, "rb").read()).hexdigest()
    recorded, launches, total = None, 0, 0
    for line in open(path):
        parts = line.split()
        if parts[:1] == ["source_sha1_gemm"]:
            recorded = parts[1]
        elif parts[:1] == ["kernel"] and parts[1].startswith(KERNEL_PREFIX[mode]):
            launches += int(parts[2])
            total += int(parts[2]) * int(parts[5])
    if recorded != sha or launches == 0:
        return None
    return total // launches


def cpu_baseline(wl, sample_rows, static=False, transform=False, lr_rank=0):
    """Oracle throughput on a bounded sample: `sample_rows` token rows through one block's linears.

    With ``static`` the W4A8 linears quantize with the oracle's static FP8 rule,
    the scale calibrated on the sample (untimed). With ``transform`` the W4A4
    linears run the oracle's transform_on path, calibrated on the sample and the
    weight (untimed, like the weight packing). With ``lr_rank`` the W4A4
    linears add the oracle's SVDQuant branch of that rank (random factors)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    table = wl.policy()
    mode_block = {0: None, 1: None}
    for b in range(wl.n_blocks):
        md = int(table[0, b])
        if mode_block[md] is None:
            mode_block[md] = b
    flops, secs = 0, 0.0
    rows = min(sample_rows, wl.m_video)
    x = synth.activation_bf16(wl.config_id, rows, wl.dim, wl.outliers, tensor_id=synth.T_X_VIDEO)
    aw_group = {}  # transform_on: joint weight maxima of the linears that read one input (as on the GPU)
    if transform and mode_block[0] is not None:
        grouped = {input_group(n) for n in SHARED_INPUT}
        for li, lin in enumerate(wl.linears):
            g = input_group(lin.name)
            if g in grouped:
                aw = oracle.hadamard_channel_amax([synth.weight_bf16(wl.config_id, lin.n, lin.k, 0, mode_block[0], li)])
                aw_group[g] = aw if g not in aw_group else np.maximum(aw_group[g], aw)
    for md, b in mode_block.items():
        if b is None:
            continue
        for li, lin in enumerate(wl.linears):
            if lin.m_role == "ffn_hidden":
                continue
            w = synth.weight_bf16(wl.config_id, lin.n, lin.k, 0, b, li)
            xs = x[:, : lin.k]
            if md == 0 and transform:
                aw = aw_group.get(input_group(lin.name))
                am, wm = oracle.smoothquant_factors(oracle.hadamard_channel_amax([xs]),
                                                    oracle.hadamard_channel_amax([w]) if aw is None else aw)
                wq, wsc = oracle.mxfp4_quantize_hadamard(w, wm)  # offline on both sides; not timed
            else:
                wq, wsc = oracle.mxfp4_quantize(w)  # offline on both sides; not timed
            amax = oracle.fp8_calibration_amax([xs]) if static else None
            t0 = time.perf_counter()
            if md == 0 and transform:
                y, _, _ = oracle.qlinear_transform(oracle.TRANSFORM_ON, xs, wq, wsc, am, epilogue=lin.epilogue)
            elif md == 0 and lr_rank:
                g = np.random.default_rng(li)
                l1t = synth.f32_to_bf16_bits((g.standard_normal((lr_rank, lin.k)) * 0.02).astype(np.float32))
                l2 = synth.f32_to_bf16_bits((g.standard_normal((lin.n, lr_rank)) * 0.02).astype(np.float32))
                ac, asc = oracle.mxfp4_quantize(xs)
                t = oracle.lowrank_down(xs, l1t)
                y = oracle.svdquant_linear_fused(md, ac, asc, wq, wsc, t, l2, None, lin.epilogue)
            elif md == 1 and static:
                ac, asc = oracle.fp8_quantize_static(xs, amax)
                y = oracle.qdq_matmul(md, ac, asc, wq, wsc, None, lin.epilogue)
            else:
                y, _, _ = oracle.qlinear(md, xs, wq, wsc, epilogue=lin.epilogue)
            secs += time.perf_counter() - t0
            flops += 2 * rows * lin.n * lin.k
            if secs > 10:
                break
        if secs > 10:
            break
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{rows} token rows through the first W4A4 and first W4A8 block's video-token linears "
                      f"(quantize{' (W4A8: static FP8)' if static else ''}"
                      f"{' (W4A4: transform_on)' if transform else ''}"
                      f"{f' (W4A4: + rank-{lr_rank} SVDQuant branch)' if lr_rank else ''} + float64 QDQ matmul), "
                      f"{flops / 1e9:.1f} GFLOP in {secs:.1f} s"}


SELECT_M = 32760  # one 480p calibration sample: 21 x 30 x 52 latent tokens (the page's 832 x 480, 81 frames)


def run_select(args, torch, mxq):
    """Calibration-driven block selection over the A14B 2-expert, 40-block model.

    The captured BF16 data of one calibration sample (synthetic inputs; every
    linear's output and the FFN hidden state from torch's bf16 matmul, which is
    the BF16 path the page compares against) are made untimed. The timed part
    is the library's block replay (OFF: plain MXFP4; ON: transform calibrated on
    the sample) with its SQNR reductions, one call per block."""
    wl = synth.workload(5)
    dev = "cuda:0"
    to_dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    m = SELECT_M
    x_video = to_dev(synth.activation_bf16(wl.config_id, m, wl.dim, wl.outliers, tensor_id=synth.T_X_VIDEO))
    x_text = to_dev(synth.activation_bf16(wl.config_id, wl.m_text, wl.dim, wl.outliers, tensor_id=synth.T_X_TEXT))
    sums_off = torch.zeros((wl.n_experts, wl.n_blocks, 2), dtype=torch.float64, device=dev)
    sums_on = torch.zeros_like(sums_off)
    ws = None
    replay_ms, flops, n_blocks = 0.0, 0, 0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    for e in range(wl.n_experts):
        for b in range(wl.n_blocks):
            lins, h = [], None
            for li, lin in enumerate(wl.linears):
                w = synth.weight_bf16_device(wl.config_id, lin.n, lin.k, e, b, li)
                if lin.m_role == "video":
                    x = x_video
                elif lin.m_role == "text":
                    x = x_text
                else:
                    x = h
                y_ref = torch.mm(x, w.t().contiguous())  # the BF16 path's output (captured)
                if lin.name == "ffn_up":  # the BF16 block's hidden state (captured)
                    h = torch.nn.functional.gelu(y_ref.float(), approximate="tanh").to(torch.bfloat16)
                lins.append((x, w, y_ref))
                flops += 2 * 2 * x.shape[0] * lin.n * lin.k  # OFF and ON GEMMs
            if ws is None:
                ws = torch.empty((mxq.replay_workspace_bytes(lins),), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            ev0.record()
            mxq.block_replay_sqnr(lins, sums_off[e, b], sums_on[e, b], ws)
            ev1.record()
            torch.cuda.synchronize()
            replay_ms += ev0.elapsed_time(ev1)
            n_blocks += 1
            del lins, h
        log(f"expert {e} replayed ({time.time() - t0:.1f}s)")
    off, on = sums_off.cpu().numpy(), sums_on.cpu().numpy()
    table = mxq.policy_select(off, on, mxq.TIER_HIGH)
    sq = lambda a: 10 * np.log10(a[..., 0] / a[..., 1])
    counts = {name: int((table == v).sum()) for name, v in (("w4a4", 0), ("w4a8", 1), ("bf16", 2),
                                                            ("transform_on", 3))}
    out = {
        "metric": "block-replay selection throughput: A14B blocks scored per second (one 480p calibration sample)",
        "value": round(n_blocks / (replay_ms * 1e-3), 3),
        "unit": "blocks/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "ms_per_block": round(replay_ms / n_blocks, 3),
        "replay_tflops": round(flops / (replay_ms * 1e-3) / 1e12, 1),
        "dtype": "mxfp4xmxfp4->fp32acc->bf16 (OFF and ON), fp64 SQNR sums",
        "data": "synthetic (seeded activations with Student-t outlier channels, N(0,0.02) weights); BF16 "
                "reference outputs from torch bf16 matmul, untimed",
        "config": {"workload": "a14b_40block_2expert_selection", "m_video": m, "m_text": wl.m_text,
                   "experts": wl.n_experts, "blocks": wl.n_blocks, "linears_per_block": len(wl.linears),
                   "tier": "high"},
        "roofline": {"bound": "mfma", "achieved": round(flops / (replay_ms * 1e-3) / 1e12, 1),
                     "peak": PEAK_TFLOPS[0], "unit": "TFLOP/s",
                     "frac": round(flops / (replay_ms * 1e-3) / 1e12 / PEAK_TFLOPS[0], 4), "traffic": None,
                     "kernel": "whole block replay (W4A4 GEMMs OFF and ON, their quantizers, maxima, reductions)"},
        "policy_counts": counts,
        "sqnr_db_off": {"min": round(float(sq(off).min()), 2), "max": round(float(sq(off).max()), 2)},
        "sqnr_db_on": {"min": round(float(sq(on).min()), 2), "max": round(float(sq(on).max()), 2)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_select_baseline(wl)
    print(json.dumps(out), flush=True)


def cpu_select_baseline(wl):
    """The oracle's block replay on a bounded sample: 128 tokens through the first block's video linears."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    rows = 128
    x = synth.activation_bf16(wl.config_id, rows, wl.dim, wl.outliers, tensor_id=synth.T_X_VIDEO)
    lins = []
    for li, lin in enumerate(wl.linears):
        if lin.m_role != "video":
            continue
        w = synth.weight_bf16(wl.config_id, lin.n, lin.k, 0, 0, li)
        y_ref = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(x) @
                                                                oracle.bf16_bits_to_f64(w).T))
        lins.append((x, w, y_ref))
        if len(lins) == 2:
            break
    t0 = time.perf_counter()
    oracle.block_replay_sums(lins)
    secs = time.perf_counter() - t0
    tokens_per_s = rows / secs
    return {"value": round(tokens_per_s, 2), "unit": "tokens/s through two linears (OFF and ON)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} token rows through the first block's first two video linears, {secs:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mx_bit_quantized_amd as mxq

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}), flush=True)
        return
    mxq.lib()
    if args.peak:
        pk = measure_peaks(torch, args.peak_seconds)
        print(json.dumps({"metric": "roofline denominators measured on this GPU", "n_gpus": 1,
                          "mfma_fp4xfp4_tflops": pk["fp4xfp4"]["tflops"], "mfma_fp4xfp8_tflops": pk["fp4xfp8"]["tflops"],
                          "spec_peak_tflops": {"fp4xfp4": PEAK_TFLOPS[0], "fp4xfp8": PEAK_TFLOPS[1]},
                          "hbm_copy_gbs": pk["copy_gbs"], "spec_hbm_gbs": PEAK_HBM_GBS, "detail": pk}), flush=True)
        return
    if args.gemm_power:
        print(json.dumps({"metric": "A14B W4A4 GEMM 75600x5120x5120 and W4A8 FFN GEMMs under sustained load: "
                                    "rate, socket power, clock",
                          "n_gpus": 1, "cases": gemm_power(torch, mxq)}), flush=True)
        return
    if args.select:
        run_select(args, torch, mxq)
        return
    wl = synth.workload(WORKLOADS[args.workload])
    shards = max(1, args.token_shards)
    if shards > 1:
        # token sharding needs no exchange: MX blocks and per-token scales are row-local
        import dataclasses
        wl = dataclasses.replace(wl, name=f"{wl.name}_tokenshard{shards}", m_video=-(-wl.m_video // shards))
    static = args.act_scale == "static"
    transform = args.transform_on
    if transform and args.svdquant_rank:
        print("--transform-on and --svdquant-rank are separate W4A4 transforms: pick one", file=sys.stderr)
        sys.exit(2)
    stack = Stack(wl, torch, mxq, static, transform, args.svdquant_rank, fuse=not args.separate_qkv)
    for _ in range(args.warmup):
        stack.step(timed=False)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with PowerSampler() as power:
        start.record()
        # per-kernel events on the last timed step only: recording them around every
        # launch slows a step by 1.4% at full size (11% at an 8-way token shard)
        for i in range(args.steps):
            stack.step(timed=i == args.steps - 1)
        end.record()
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    tflops = wl.total_flops() / (ms_per_step * 1e-3) / 1e12

    # per-kernel aggregates from the per-launch events
    agg = {}
    for kind, mode, fl, by, e0, e1 in stack.records:
        ms = e0.elapsed_time(e1)
        a = agg.setdefault((kind, mode), {"ms": 0.0, "flops": 0, "bytes": 0, "launches": 0})
        a["ms"] += ms
        a["flops"] += fl
        a["bytes"] += by
        a["launches"] += 1
    kernels = {}
    for (kind, mode), a in agg.items():
        name = f"{kind}_{'w4a4' if mode == 0 else 'w4a8'}"
        d = {"launches_per_step": a["launches"], "avg_us": round(1e3 * a["ms"] / a["launches"], 2),
             "share_of_step": round(a["ms"] / ms_per_step, 4)}
        if kind == "gemm":
            d["tflops"] = round(a["flops"] / (a["ms"] * 1e-3) / 1e12, 1)
            d["frac_of_peak"] = round(d["tflops"] / PEAK_TFLOPS[mode], 4)
        else:
            d["gbs"] = round(a["bytes"] / (a["ms"] * 1e-3) / 1e9, 1)
            d["frac_of_hbm"] = round(d["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = d
    dom = max((k for k in agg if k[0] == "gemm"), key=lambda k: agg[k]["ms"])
    a = agg[dom]
    achieved = a["flops"] / (a["ms"] * 1e-3) / 1e12
    tag = [k for k, v in WORKLOADS.items() if v == wl.config_id][0] + ("_static" if static else "") + \
        ("_transform" if transform else "") + (f"_svdquant{args.svdquant_rank}" if args.svdquant_rank else "") + \
        (f"_tokenshard{shards}" if shards > 1 else "")
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS[dom[1]], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[dom[1]], 4),
                "traffic": profiled_traffic(tag, dom[1]),
                "kernel": KERNEL_SYMBOL[dom[1]],
                "avg_launch_us": round(1e3 * a["ms"] / a["launches"], 1),
                "flop_per_launch": a["flops"] // a["launches"]}
    if not args.no_peak_probe:
        # the same instruction with nothing else running, on random operands, at
        # the clock the board's power cap allows (spec peak assumes 2.4 GHz)
        pk = measure_peaks(torch, args.peak_seconds)
        mp = pk["fp4xfp4" if dom[1] == 0 else "fp4xfp8"]
        roofline["measured_peak"] = {"value": mp["tflops"], "unit": "TFLOP/s", "clock_ghz": mp["clock_ghz"],
                                     "socket_w": mp["socket_w"],
                                     "kind": "register-only scaled MFMA, random operands, one wave per SIMD on every CU"}
        roofline["frac_of_measured_peak"] = round(achieved / mp["tflops"], 4)
        roofline["hbm_copy_gbs"] = pk["copy_gbs"]
    modes = set(int(v) for v in stack.policy_table.flat)
    out = {
        "metric": METRIC,
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak" if shards == 1 else "strong",
        "vs_baseline": None,
        "dtype": "+".join(x for x, md in (("mxfp4xmxfp4", 0), ("fp8e4m3xmxfp4", 1)) if md in modes) + "->fp32acc->bf16",
        "data": "synthetic (seeded activations with Student-t outlier channels; N(0,0.02) weights, RTN MXFP4"
                + ("; static FP8 scales calibrated, untimed, on the same inputs" if static else "")
                + ("; transform_on factors calibrated, untimed, on the same inputs and weights" if transform else "")
                + ")",
        "config": {"workload": wl.name, "m_video": wl.m_video, "m_text": wl.m_text, "dim": wl.dim, "ffn": wl.ffn,
                   "experts": wl.n_experts, "blocks": wl.n_blocks,
                   "w4a8_blocks": int((stack.policy_table == 1).sum()),
                   "w4a8_activations": "fp8_static_per_tensor" if static else "fp8_per_token",
                   "w4a4_transform": "hadamard128+smoothquant" if transform else
                   (f"svdquant_rank{args.svdquant_rank}" if args.svdquant_rank else "none"),
                   "linears_per_block": len(wl.linears), "gemms_per_block": len(stack.lins),
                   "tflop_per_step": round(wl.total_flops() / 1e12, 2),
                   **({"token_shards": shards} if shards > 1 else {})},
        "roofline": roofline,
        "power": power.summary(),
        "kernels": kernels,
        "weight_pack_gbs": round(stack.pack_gbs, 1),
        # high-water mark of device memory over the run (every buffer is a torch
        # allocation: the library allocates none)
        "peak_device_gib": round(torch.cuda.max_memory_allocated() / 2 ** 30, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_rows, static, transform, args.svdquant_rank)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
