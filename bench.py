"""Benchmark: FP8 scaled-GEMM TFLOP/s on one MI355X.

Workload: per-tensor E4M3 x E4M3 scaled GEMM d = (a * s_a) @ (b * s_b)^T with
N = K = 4096 and M in {16, 64, 256, 1024, 2048, 8192}, slow accumulation
(128-element chunks promoted into fp32), bf16 output, seeded synthetic
Gaussian inputs (x = z * 240 / max|z| per tensor). One step = one GEMM at each
of the six M values. Inputs stay resident in HBM; every M cycles through
enough distinct buffer sets (row rotations of the seeded data, at least
512 MB per M) that the 256 MB Infinity Cache cannot hold them, so the small-M
runs are measured against HBM rather than cache.

Prints one JSON line. `value` = the step's total flops / the step's time.
`roofline` describes the dominant kernel (the M = 8192 GEMM), timed with HIP
events on the stream it runs on. Its products run on the bf16 MFMA (each FP8
operand is converted exactly to bf16 in registers: the FP8 MFMA's own
accumulation is not accurate enough for the required 2^-20 sum|a b| bound), so
the roofline peak is the dense bf16 MFMA rate; the per-M lines also give the
fraction of the FP8 MFMA peak that the metric names. `traffic` is the HBM bytes
per launch of that kernel from committed rocprofv3 counters, reported only while
the kernel sources are the ones the counters were taken on.

Method (after "mmaemu backends", Benchmarks, Method):
 - exactness gate before timing: every M's output on the first buffer set is
   compared with the CPU oracle on rows 0 .. min(M, 64) - 1 plus 64 seeded rows,
   all columns; any output outside the tolerance stops the run (exit 1) after
   printing the first bad elements. The oracle's time on those rows is the
   `cpu_baseline` (all host cores, and one thread);
 - warm-up: the requested untimed steps, then more untimed steps until at least
   1.5 s have passed (`warmup_s`), so that the clock has settled;
 - the requested K steps are timed (`value`); then interleaved windows of at
   least 1.0 s each run the same step loop, and their median is reported with
   the GPU clock sampled every 200 ms meanwhile (`method`), as a rate per clock
   (flop per clock per CU) and as a fraction of the bf16 MFMA peak at that clock.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

MS = (16, 64, 256, 1024, 2048, 8192)
N = K = 4096
PEAK_FP8_TFLOPS = 5033.0      # MI355X dense FP8 MFMA: 256 CUs x 8192 flop/clk x 2.4 GHz
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CUs x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP4_TFLOPS = 10066.0     # MI355X dense FP4 MFMA: 4x the bf16 rate
COUNTERS = os.path.join(ROOT, "profiles", "gemm_tile_M8192_N4096_K4096_slow_counters.md")
KERNEL_SOURCES = [os.path.join(ROOT, "block_scaled_gemm_amd", "csrc", f) for f in ("mm_kernels.hpp", "mm_launch.hpp")]
ROTATION_BYTES = 512 << 20    # 2x the Infinity Cache
METRIC = "FP8 scaled-GEMM TFLOP/s and % of MI355X FP8 MFMA peak, M=16..8192"
# kernel the library dispatches for each M of the benchmark (N = K = 4096, per-tensor)
KERNEL_AT = {16: "gemm_skinny", 64: "gemm_skinny_k", 256: "gemm_ksplit"}


def gemm_bytes(M):
    # algorithmic bytes: A + B read once, D (bf16) written once, two fp32 scales
    return M * K + N * K + 2 * M * N + 8


def gemm_flops(M):
    return 2.0 * M * N * K


def kernel_sources_digest():
    """sha256 of the kernel sources with their comments, trailing blanks and
    empty lines removed: a counter summary holds while the code it measured is
    unchanged, whatever the comments say."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()


def counters_profile():
    """The committed counter summary of the M = 8192 kernel, or None when the
    kernel code changed since it was taken (its figures no longer apply)."""
    import re
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    digest = re.search(r"kernel_sources_sha256: ([0-9a-f]{64})", text)
    if not digest or digest.group(1) != kernel_sources_digest():
        return None
    return text


def measured_traffic():
    """HBM bytes per launch of the M = 8192 kernel from the committed counter
    summary, or None."""
    import re
    text = counters_profile()
    traffic = re.search(r"traffic_bytes_per_launch: (\d+)", text) if text else None
    return int(traffic.group(1)) if traffic else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_sets(M, torch, dev, datagen):
    d = datagen.set_gauss_n4096(M, N, K)
    a0 = torch.from_numpy(d["a"]).to(dev)
    b0 = torch.from_numpy(d["b"]).to(dev)
    sa = torch.tensor([d["scale_a"]], dtype=torch.float32, device=dev)
    sb = torch.tensor([d["scale_b"]], dtype=torch.float32, device=dev)
    n = max(2, math.ceil(ROTATION_BYTES / gemm_bytes(M)))
    sets = []
    for i in range(n):
        a = torch.roll(a0, shifts=(i * 7) % max(M, 1), dims=0).contiguous()
        b = torch.roll(b0, shifts=i * 131, dims=0).contiguous()
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        sets.append((a, b, out))
    return dict(sets=sets, sa=sa, sb=sb)


def launch(mm, M, s, S, stream):
    a, b, out = s
    st = mm.mm_scaled_gemm(M, N, K, a.data_ptr(), mm.MM_F8_E4M3FN, K, b.data_ptr(), mm.MM_F8_E4M3FN, K,
                           S["sa"].data_ptr(), mm.MM_SCALE_TENSOR, S["sb"].data_ptr(), mm.MM_SCALE_TENSOR, 0,
                           out.data_ptr(), mm.MM_BF16, N, 0, stream)
    if st != mm.MM_OK:
        raise RuntimeError(f"mm_scaled_gemm failed: {mm.mm_last_error()}")


def gate_rows(M):
    """Rows the exactness gate checks: 0 .. min(M, 64) - 1 plus 64 seeded rows of the rest."""
    import numpy as np
    first = np.arange(min(M, 64))
    if M <= 64:
        return first
    rest = np.random.default_rng(1000 + M).choice(np.arange(64, M), size=min(64, M - 64), replace=False)
    return np.unique(np.concatenate([first, rest]))


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_and_gate(outputs, ms):
    """The CPU oracle leg. For every M it computes the oracle (exact float64 sums, untuned) on the gate rows
    of the first buffer set, timed on all host cores and again on one thread, and compares the GPU's output of
    that buffer set with it element by element (tests/compare.py tolerances). Returns (cpu_baseline, gate);
    gate["passed"] is False at the first M with an output out of tolerance, whose message names it."""
    import numpy as np
    import compare
    import datagen
    import oracle
    threads = host_cores()
    flops, secs, secs1, checked = 0.0, 0.0, 0.0, 0
    gate = {"passed": True, "rows": "0..min(M,64)-1 plus 64 seeded rows, all columns", "outputs_checked": 0}
    for M in ms:
        d = datagen.set_gauss_n4096(M, N, K)
        rows = gate_rows(M)
        args = (d["a"], 0, d["b"], 0, d["scale_a"], 0, d["scale_b"], 0, oracle.BF16)
        t = time.perf_counter()
        value, sabs, bits = oracle.scaled_gemm(*args, accum=oracle.ACC_EXACT, rows=rows, threads=threads)
        secs += time.perf_counter() - t
        t = time.perf_counter()
        oracle.scaled_gemm(*args, accum=oracle.ACC_EXACT, rows=rows, threads=1)
        secs1 += time.perf_counter() - t
        flops += 2.0 * rows.size * N * K
        gpu = outputs[M][rows]
        try:
            compare.check(gpu, value, sabs, bits, compare.BF16, f"exactness gate M={M}")
        except AssertionError as e:
            gate["passed"] = False
            gate["message"] = str(e)
            break
        checked += gpu.size
    gate["outputs_checked"] = checked
    base = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the exactness gate's rows of the benchmark step: M in {list(ms)}, N=K=4096, "
                      f"rows 0..min(M,64)-1 plus 64 seeded rows of each M ({flops:.3g} flop, exact float64 "
                      f"sums), {secs:.2f} s on {threads} threads",
            "value_1thread": flops / secs1 / 1e12, "seconds_1thread": round(secs1, 2),
            "cpu_model": cpu_model()}
    return base, gate


class ClockSampler:
    """Samples the GPU's graphics clock every 200 ms in a background thread through the amdsmi library (the
    library behind amd-smi); `mean_mhz()` is None when no sample could be taken."""

    def __init__(self, period=0.2):
        import threading
        self.period = period
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            h = amdsmi.amdsmi_get_processor_handles()[0]
            while not self._stop.is_set():
                clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX).get("clk")
                if isinstance(clk, (int, float)) and clk > 0:
                    self.samples.append(float(clk))
                self._stop.wait(self.period)
            amdsmi.amdsmi_shut_down()
        except Exception as e:  # no library, no permission, no device: report no clock
            self.error = f"{type(e).__name__}: {e}"

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join(timeout=5)

    def mean_mhz(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


# ------------------------------------------------------------------ other workloads
# Single-GEMM timings of the remaining configurations, for their own roofline
# lines (`--workload NAME`); the default run above is the benchmark itself.

OTHER = {
    "block": "E4M3 1x128 / 128x128 block-scaled GEMM, M=4096, N=14336, K=4096, bf16 out",
    "mx_amax": "batched E4M3 GEMM with power-of-two scales per 32 K, L=8, M=N=2048, K=8192, f32 C + amax + index",
    "e4m3_out": "E4M3 GEMM, M=8192, N=28672, K=8200 (lda 8200), slow, E4M3 out via scale_result=1/16",
    "e5m2_f16": "E5M2 GEMM, M=8192, N=28672, K=8200 (lda 8200), slow, f16 out",
    "shard_e4m3_out": "one GPU's share of the E4M3-out GEMM split over 8 GPUs by columns: M=8192, N=3584, K=8200 "
                      "(lda 8200), slow, E4M3 out via scale_result=1/16",
    "shard_mx_l1": "one GPU's share of the batched MX GEMM + amax split over 8 GPUs by batch item: L=1, M=N=2048, "
                   "K=8192, power-of-two scales per 32 K, f32 C + amax + index",
    "block_bias": "E4M3 1x128 / 128x128 block-scaled GEMM + bf16 bias [N], M=4096, N=14336, K=4096, bf16 out",
    "bmm": "batched per-tensor E4M3 GEMM, L=8, M=N=2048, K=4096, slow, bf16 out",
    "bmm_kn": "batched per-tensor E4M3 GEMM with b as [L, K, N] (transposed per call), L=8, M=N=2048, K=4096, "
              "slow, bf16 out",
    "mx_atom": "batched E4M3 GEMM with E8M0 factors per 32 K in the page-native atom layout, L=8, M=N=2048, "
               "K=8192, f32 C + amax + index",
    "mx_fp4": "batched FP4 (E2M1) GEMM with E8M0 factors per 32 K in the page-native atom layout, L=8, "
              "M=N=2048, K=8192, f32 C + amax + index",
    "mx_nvfp4": "batched FP4 (E2M1) GEMM with E4M3 factors per 16 K in the page-native atom layout, L=8, "
                "M=N=2048, K=8192, f32 C + amax + index",
    "grouped": "grouped per-tensor E4M3 GEMM (NT), 8 groups of ragged sizes packing 8192 rows, N=K=4096, slow, "
               "bf16 out",
    "grouped_nn": "grouped per-tensor E4M3 GEMM (NN, b [G, K, N] packed per call), 8 groups of ragged sizes "
                  "packing 8192 rows, N=K=4096, slow, bf16 out",
    "grouped_tn": "grouped per-tensor E4M3 GEMM (TN, the groups split the contraction, both operands packed per "
                  "call), 8 groups of ragged sizes packing 8192 rows, blocks [8, 4096, 4096], slow, bf16 out",
}


def run_other(name, steps, warmup, settle_s=1.5):
    import torch
    import block_scaled_gemm_amd as mm
    import datagen
    import numpy as np
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.time()
    if name in ("block", "block_bias"):
        d = datagen.set_block_scaled_4096x14336x4096()
        M, K = d["a"].shape; N = d["b"].shape[0]; L = 1
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        sa = torch.from_numpy(d["scale_a"]).to(dev); sb = torch.from_numpy(d["scale_b"]).to(dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        out_bytes = 2

        if name == "block":
            def launch():
                return mm.mm_scaled_gemm(M, N, K, a.data_ptr(), mm.MM_F8_E4M3FN, K, b.data_ptr(), mm.MM_F8_E4M3FN,
                                         K, sa.data_ptr(), mm.MM_SCALE_1x128, sb.data_ptr(), mm.MM_SCALE_128x128, 0,
                                         out.data_ptr(), mm.MM_BF16, N, 0, stream)
            scale_bytes = 4 * (sa.numel() + sb.numel())
        else:
            bias = torch.from_numpy(datagen.bias_bf16_bits(N).view(np.int16)).to(dev)

            def launch():
                return mm.mm_scaled_gemm_bias(M, N, K, a.data_ptr(), mm.MM_F8_E4M3FN, K, b.data_ptr(),
                                              mm.MM_F8_E4M3FN, K, sa.data_ptr(), mm.MM_SCALE_1x128, sb.data_ptr(),
                                              mm.MM_SCALE_128x128, bias.data_ptr(), out.data_ptr(), mm.MM_BF16, N, 0,
                                              stream)
            scale_bytes = 4 * (sa.numel() + sb.numel()) + 2 * N
    elif name == "bmm":
        d = datagen.set_bmm_l8_2048x2048x4096()
        L, M, K = d["a"].shape; N = d["b"].shape[1]
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        sa = torch.tensor([float(d["scale_a"])], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(d["scale_b"])], dtype=torch.float32, device=dev)
        out = torch.empty((L, M, N), dtype=torch.bfloat16, device=dev)
        out_bytes = 2

        def launch():
            return mm.mm_scaled_gemm_batched(L, M, N, K, a.data_ptr(), mm.MM_F8_E4M3FN, K, M * K, b.data_ptr(),
                                             mm.MM_F8_E4M3FN, K, N * K, sa.data_ptr(), sb.data_ptr(), 0,
                                             out.data_ptr(), mm.MM_BF16, N, M * N, 0, stream)
        scale_bytes = 8
    elif name == "bmm_kn":
        d = datagen.set_bmm_l8_2048x2048x4096()
        L, M, K = d["a"].shape; N = d["b"].shape[1]
        a = torch.from_numpy(d["a"]).to(dev)
        b = torch.from_numpy(np.ascontiguousarray(d["b"].transpose(0, 2, 1))).to(dev)  # [L, K, N]
        bt = torch.empty((L, N, K), dtype=torch.uint8, device=dev)
        sa = torch.tensor([float(d["scale_a"])], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(d["scale_b"])], dtype=torch.float32, device=dev)
        out = torch.empty((L, M, N), dtype=torch.bfloat16, device=dev)
        out_bytes = 2

        def launch():
            st = mm.mm_transpose_u8(L, K, N, b.data_ptr(), N, K * N, bt.data_ptr(), K, N * K, stream)
            if st != mm.MM_OK:
                return st
            return mm.mm_scaled_gemm_batched(L, M, N, K, a.data_ptr(), mm.MM_F8_E4M3FN, K, M * K, bt.data_ptr(),
                                             mm.MM_F8_E4M3FN, K, N * K, sa.data_ptr(), sb.data_ptr(), 0,
                                             out.data_ptr(), mm.MM_BF16, N, M * N, 0, stream)
        scale_bytes = 8
    elif name in ("mx_amax", "shard_mx_l1"):
        d = datagen.set_mx_l8_2048x2048x8192()
        if name == "shard_mx_l1":  # batch item 0: what one of 8 GPUs computes when the batch is split
            d = {k: (v[:1] if k in ("a", "b", "sfa", "sfb") else v) for k, v in d.items()}
        L, M, K = d["a"].shape; N = d["b"].shape[1]
        a = torch.from_numpy(np.ascontiguousarray(d["a"])).to(dev)
        b = torch.from_numpy(np.ascontiguousarray(d["b"])).to(dev)
        sfa = torch.from_numpy(np.ascontiguousarray(d["sfa"])).to(dev)
        sfb = torch.from_numpy(np.ascontiguousarray(d["sfb"])).to(dev)
        c = torch.empty((L, M, N), dtype=torch.float32, device=dev)
        amax = torch.empty((1,), dtype=torch.float32, device=dev)
        idx = torch.empty((1,), dtype=torch.int64, device=dev)
        out_bytes = 4

        def launch():
            return mm.mm_blockscaled_gemm_amax(M, N, K, L, a.data_ptr(), b.data_ptr(), mm.MM_F8_E4M3FN,
                                               sfa.data_ptr(), sfb.data_ptr(), 32, c.data_ptr(), mm.MM_F32,
                                               amax.data_ptr(), idx.data_ptr(), stream)
        scale_bytes = 4 * (sfa.numel() + sfb.numel()) + 12
    elif name == "grouped":
        d = datagen.set_grouped_8x8192x4096x4096()
        M, K = d["a"].shape; N = d["b"].shape[1]; L = 1; G = d["b"].shape[0]
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        gs = torch.from_numpy(d["sizes"]).to(dev); go = torch.from_numpy(d["offsets"]).to(dev)
        sa = torch.tensor([float(d["scale_a"])], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(d["scale_b"])], dtype=torch.float32, device=dev)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        out_bytes = 2

        def launch():
            return mm.mm_scaled_gemm_grouped(M, N, K, G, a.data_ptr(), mm.MM_F8_E4M3FN, K, b.data_ptr(),
                                             mm.MM_F8_E4M3FN, K, N * K, gs.data_ptr(), go.data_ptr(), sa.data_ptr(),
                                             sb.data_ptr(), 0, out.data_ptr(), mm.MM_BF16, N, 0, stream)
        # every group's b is read: G N K bytes in place of N K
        scale_bytes = 8 + 8 * G + (G - 1) * N * K
    elif name in ("grouped_nn", "grouped_tn"):
        tn = name == "grouped_tn"
        d = datagen.set_grouped_layout(8, 8192, 4096, 4096, 0, tn, False, config=9)
        S = d["a"].shape[0]; G = d["sizes"].size; N = K = N0 = K0 = 4096
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        gs = torch.from_numpy(d["sizes"]).to(dev); go = torch.from_numpy(d["offsets"]).to(dev)
        sa = torch.tensor([float(d["scale_a"])], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(d["scale_b"])], dtype=torch.float32, device=dev)
        out = torch.empty((G, N, K) if tn else (S, N), dtype=torch.bfloat16, device=dev)
        st, ws_bytes = mm.mm_grouped_workspace_bytes(S, N, K, G, int(tn), 0)
        ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        out_bytes = 2

        def launch():
            return mm.mm_scaled_gemm_grouped_layout(S, N0, K0, G, int(tn), 0, a.data_ptr(), mm.MM_F8_E4M3FN,
                                                    d["a"].shape[1], b.data_ptr(), mm.MM_F8_E4M3FN, d["b"].shape[-1],
                                                    0 if tn else K0 * N0, gs.data_ptr(), go.data_ptr(),
                                                    sa.data_ptr(), sb.data_ptr(), 0, out.data_ptr(), mm.MM_BF16,
                                                    K0 if tn else N0, N0 * K0 if tn else 0, ws.data_ptr(), ws_bytes,
                                                    0, stream)
        if tn:
            # as one GEMM of [N, S] by [S, K] (flops 2 N K S) whose output is G blocks of [N, K]
            L, M, N, K = 1, N, K, S
            scale_bytes = 8 + 8 * G + (G - 1) * M * N * out_bytes
        else:
            L, M = 1, S
            scale_bytes = 8 + 8 * G + (G - 1) * N * K  # every group's b is read
    elif name in ("mx_atom", "mx_fp4", "mx_nvfp4"):
        d = {"mx_atom": datagen.set_mx_atom_l8_2048x2048x8192, "mx_fp4": datagen.set_fp4_l8_2048x2048x8192, "mx_nvfp4": datagen.set_nvfp4_l8_2048x2048x8192}[name]()
        L, M, K = d["a"].shape; N = d["b"].shape[1]
        ab_type = mm.MM_F8_E4M3FN if name == "mx_atom" else mm.MM_F4_E2M1
        K = K if name == "mx_atom" else 2 * K
        sf_type, sf_vec = (mm.MM_SF_E4M3FN, 16) if name == "mx_nvfp4" else (mm.MM_SF_E8M0, 32)
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        sfa = torch.from_numpy(d["sfa"]).to(dev); sfb = torch.from_numpy(d["sfb"]).to(dev)
        c = torch.empty((L, M, N), dtype=torch.float32, device=dev)
        amax = torch.empty((1,), dtype=torch.float32, device=dev)
        idx = torch.empty((1,), dtype=torch.int64, device=dev)
        out_bytes = 4

        def launch():
            return mm.mm_blockscaled_gemm_amax_atom(M, N, K, L, a.data_ptr(), b.data_ptr(), ab_type,
                                                    sfa.data_ptr(), sfb.data_ptr(), sf_type, sf_vec, c.data_ptr(),
                                                    mm.MM_F32, amax.data_ptr(), idx.data_ptr(), stream)
        scale_bytes = sfa.numel() + sfb.numel() + 12
    else:
        e4 = name in ("e4m3_out", "shard_e4m3_out")
        d = datagen.set_e4m3_out_8192x28672x8200() if e4 else datagen.set_e5m2_f16_8192x28672x8200()
        if name == "shard_e4m3_out":  # the first 3584 columns: what one of 8 GPUs computes when N is split
            d = dict(d, b=np.ascontiguousarray(d["b"][:3584]))
        M, K = d["a"].shape; N = d["b"].shape[0]; L = 1
        fa = mm.MM_F8_E4M3FN if e4 else mm.MM_F8_E5M2
        a = torch.from_numpy(d["a"]).to(dev); b = torch.from_numpy(d["b"]).to(dev)
        sa = torch.tensor([float(d["scale_a"])], dtype=torch.float32, device=dev)
        sb = torch.tensor([float(d["scale_b"])], dtype=torch.float32, device=dev)
        sr = torch.tensor([float(d.get("scale_result", 1.0))], dtype=torch.float32, device=dev)
        dt = mm.MM_F8_E4M3FN if e4 else mm.MM_F16
        out_bytes = 1 if e4 else 2
        out = torch.empty((M * N * out_bytes,), dtype=torch.uint8, device=dev)

        def launch():
            return mm.mm_scaled_gemm(M, N, K, a.data_ptr(), fa, K, b.data_ptr(), fa, K, sa.data_ptr(),
                                     mm.MM_SCALE_TENSOR, sb.data_ptr(), mm.MM_SCALE_TENSOR,
                                     sr.data_ptr() if e4 else 0, out.data_ptr(), dt, N, 0, stream)
        scale_bytes = 12
    torch.cuda.synchronize()
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s")
    for _ in range(warmup):
        if launch() != mm.MM_OK:
            raise RuntimeError(mm.mm_last_error())
    torch.cuda.synchronize()
    settle_steps, settle_secs = settle(lambda i: launch(), settle_s) if settle_s > 0 else (0, 0.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    flops = 2.0 * L * M * N * K
    tf = flops / us / 1e6
    op_bytes = 0.5 if name in ("mx_fp4", "mx_nvfp4") else 1.0  # operand bytes per element (FP4: two per byte)
    # FP4 with E8M0 factors runs on the scaled FP4 MFMA (peak 4x bf16); every other workload on the bf16 MFMA
    peak, peak_note = (PEAK_FP4_TFLOPS, "dense FP4 MFMA") if name == "mx_fp4" else \
        (PEAK_BF16_TFLOPS, "dense bf16 MFMA (operands converted exactly in registers)")
    nbytes = L * ((M + N) * K * op_bytes + M * N * out_bytes) + scale_bytes
    result = {
        "metric": f"{OTHER[name]}: TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "warmup_s": round(settle_secs, 3), "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "data": "synthetic",
        "config": {"workload": OTHER[name], "L": L, "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tf / peak, 4), "peak_unit_note": peak_note,
                     "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "hbm_gbs_algorithmic": round(nbytes / us / 1e3, 1)},
    }
    print(json.dumps(result), flush=True)


def counter_clock_ghz():
    """The clock the committed counter run measured for the M = 8192 kernel (GRBM_GUI_ACTIVE over the kernel
    time), or None."""
    import re
    text = counters_profile()
    m = re.search(r"counter_clock_ghz: ([0-9.]+)", text) if text else None
    return float(m.group(1)) if m else None


def settle(step, min_s):
    """Untimed steps until at least min_s seconds have passed; returns (steps, seconds)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while True:
        step(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= min_s:
                return n, time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before the settling phase")
    ap.add_argument("--settle-s", type=float, default=1.5,
                    help="untimed steps after --warmup until this many seconds have passed (the clock settles)")
    ap.add_argument("--windows", type=int, default=5, help="timed windows of the pages' method (median)")
    ap.add_argument("--window-s", type=float, default=1.0, help="minimum length of each window")
    ap.add_argument("--only-m", type=int, default=0, help="run only this M (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg, and with it the exactness gate (profiler runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device (reads and writes that many bytes) so that "
                         "profiler byte counters can be scaled against a kernel of known traffic")
    ap.add_argument("--workload", choices=sorted(OTHER), default=None,
                    help="time one of the other configurations instead of the benchmark step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the GEMM runs on one GPU; --gpus {args.gpus} is not supported (across GPUs the "
              "output tiles would be split by N or by the batch L, with one all-reduce of the amax)",
              file=sys.stderr)
        sys.exit(2)
    if args.workload:
        run_other(args.workload, args.steps if args.steps != 200 else 100, args.warmup if args.warmup != 100 else 50,
                  args.settle_s)
        return

    import torch
    import block_scaled_gemm_amd as mm
    import datagen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy} MiB read, {args.calibrate_copy} MiB written")
        del src, dst
    ms = (args.only_m,) if args.only_m else MS
    t0 = time.time()
    data = {M: make_sets(M, torch, dev, datagen) for M in ms}
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: " + ", ".join(f"M={M}: {len(data[M]['sets'])} sets" for M in ms))
    stream = torch.cuda.current_stream().cuda_stream
    dominant = max(ms)
    flops_step = sum(gemm_flops(M) for M in ms)

    # exactness gate (and the CPU oracle leg) before any timing
    base = gate = None
    if not args.no_cpu_baseline and not args.only_m:
        outputs = {}
        for M in ms:
            S = data[M]
            launch(mm, M, S["sets"][0], S, stream)
        torch.cuda.synchronize()
        for M in ms:
            outputs[M] = data[M]["sets"][0][2].view(torch.int16).cpu().numpy().view("uint16")
        log("exactness gate: oracle on the gate rows of every M ...")
        base, gate = cpu_baseline_and_gate(outputs, ms)
        if not gate["passed"]:
            log(gate["message"])
            print(json.dumps({"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "gate": gate}),
                  flush=True)
            sys.exit(1)
        log(f"exactness gate passed: {gate['outputs_checked']} outputs; oracle {base['value']:.4f} TFLOP/s on "
            f"{base['cores']} threads, {base['value_1thread']:.5f} on one")

    def step(i, ev=None):
        for M in ms:
            S = data[M]
            s = S["sets"][i % len(S["sets"])]
            if ev is not None and M == dominant:
                ev[0].record()
                launch(mm, M, s, S, stream)
                ev[1].record()
            else:
                launch(mm, M, s, S, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    settle_steps, settle_s = settle(lambda i: step(args.warmup + i), args.settle_s) if args.settle_s > 0 else (0, 0.0)
    log(f"settled: {args.warmup} warm-up steps, then {settle_steps} more over {settle_s:.2f} s")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    dom_us = 1e3 * sum(a.elapsed_time(b) for a, b in evs) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step; M={dominant} kernel {dom_us:.2f} us")

    # the pages' windows: interleaved windows of at least window_s seconds of the same step loop, median,
    # with the graphics clock sampled meanwhile
    windows = []
    sampler = ClockSampler().start()
    for w in range(args.windows):
        n = max(1, int(args.window_s / max(ms_step * 1e-3, 1e-6)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        while True:
            torch.cuda.synchronize()
            e0.record()
            for i in range(n):
                step(i)
            e1.record()
            torch.cuda.synchronize()
            el = e0.elapsed_time(e1) * 1e-3
            if el >= args.window_s:
                break
            n = int(n * args.window_s / max(el, 1e-6) * 1.1) + 1
        windows.append(flops_step * n / el / 1e12)
    sampler.stop()
    med = sorted(windows)[len(windows) // 2] if windows else None
    clk = sampler.mean_mhz()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    method = {"windows_tflops": [round(w, 1) for w in windows], "median_tflops": round(med, 2) if med else None,
              "window_s": args.window_s, "clock_mhz_mean": round(clk, 1) if clk else None,
              "clock_samples": len(sampler.samples), "cus": cus}
    if clk:
        method["flop_per_clk_per_cu"] = round(med * 1e12 / (clk * 1e6 * cus), 1)
        method["frac_bf16_peak_at_clock"] = round(med * 1e12 / (clk * 1e6 * cus * 4096), 4)
    if sampler.error:
        method["clock_error"] = sampler.error
    log(f"windows: {method['windows_tflops']} TFLOP/s, median {method['median_tflops']}; clock {clk} MHz")

    # per-M breakdown (each M alone, same rotation)
    per_m = {}
    for M in ms:
        S = data[M]
        reps = max(50, min(2000, int(2e5 / max(gemm_flops(M) / 4e12 * 1e6, 1))))
        for i in range(10):
            launch(mm, M, S["sets"][i % len(S["sets"])], S, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            launch(mm, M, S["sets"][i % len(S["sets"])], S, stream)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        tf = gemm_flops(M) / us / 1e6
        gbs = gemm_bytes(M) / us / 1e3
        per_m[str(M)] = {"us": round(us, 3), "tflops": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                         "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                         "hbm_gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                         "kernel": KERNEL_AT.get(M, "gemm_tile")}
        log(f"M={M}: {us:.2f} us, {tf:.1f} TFLOP/s ({100 * tf / PEAK_FP8_TFLOPS:.1f}% of FP8 peak, "
            f"{100 * tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak), {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% HBM)")

    achieved = gemm_flops(dominant) / dom_us / 1e6
    result = {
        "metric": METRIC,
        "value": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(settle_s, 3),
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 in, bf16 mfma, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "per-tensor E4M3 x E4M3 scaled GEMM, N=K=4096, M in {16,64,256,1024,2048,8192}, "
                               "slow accumulation, bf16 out", "M": list(ms), "N": N, "K": K,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if dominant == 8192 else None,
                     "peak_unit_note": "dense bf16 MFMA (FP8 operands converted exactly in registers)",
                     "frac_of_fp8_peak": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "kernel": f"{KERNEL_AT.get(dominant, 'gemm_tile')} M={dominant} N=K=4096",
                     "kernel_us": round(dom_us, 3),
                     "clock_ghz_counters": counter_clock_ghz() if dominant == 8192 else None},
        "method": method,
        "per_m": per_m,
    }
    if gate is not None:
        result["gate"] = gate
        result["cpu_baseline"] = base
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
