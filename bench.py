"""Throughput of the FlashAttention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one launch of the whole forward (scores, masks, online softmax,
P V, normalisation, LSE) over one batch: B=4, H=16, N=4096, d=128 bf16,
N(0,1) inputs, scale 1/sqrt(d), non-causal (the pages' N=4096, d=128 example
shape, in bf16).  The causal variant of the same shape (1% of key rows x8)
is timed too and reported in the "causal" object.  Inputs are resident in
HBM before timing starts.

Prints one JSON line with the headline metric (TFLOP/s, 4 B H N^2 d FLOPs,
halved for causal), the matrix-core roofline of the kernel (dense bf16 peak
of MI355X, 2.5 PFLOP/s), and the float64 CPU oracle timed on the host's cores
over a bounded sample of the same workload.

--profile-run launches a copy kernel of known size and then the forward a few
times, without timing, for rocprofv3 counter collection (HBM bytes).

--sweep times the same non-causal bf16 workload at every tile shape of the
tile-size sweep (query rows x keys in {64, 128, 256} x {32, 64, 128}, the
per-tile kernel of each shape) and prints a table with each kernel's
registers, spills, LDS bytes and occupancy beside the working set of
"FlashAttention Memory Model" Q3 (Q, K, V, O and S tiles in 16 bits).
--summarize l2 DIR reads a rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum run of it.

--backward times only the backward pass (include/fa_bwd.h) on the same
shape, non-causal and causal (after the copy kernel, for counter runs); the
default line carries the same figures in its "backward" object.

--configs times the forward (launch mean) and, for 16-bit inputs, the
backward on every named workload, one JSON line each, with the issue ceiling
of the workload's head dimension (alu_peak: the matrix work and the softmax
of the key loop co-issued on every SIMD, measured by the issue-rate probe of
include/fa_probe.h at the start of the run) and the fraction of it reached
(alu_frac).

--issue-probe prints the probe's time per instruction per SIMD for each
instruction mix of the key loop, and the ceilings they imply.

--split times the split-KV forward (fa_fwd_split, 2-16 key ranges) against
the plain launch on few-head long sequences (bf16, d = 128, non-causal and
causal).

--standard times the standard forward of include/fa_standard.h (S and P
materialised in HBM) on the same workload, after the copy kernel of
--profile-run, so that rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of it give
its HBM bytes per kernel for comparison with the tiled forward.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd TFLOP/s at N=4096 d=128 bf16 (causal and non-causal), % MFMA peak"
KERNEL_SOURCES = ("tiled_exact_attention_fwd_amd/csrc/fa_fwd_kernels.h",
                  "tiled_exact_attention_fwd_amd/csrc/fa_fwd_launch.h",
                  "tiled_exact_attention_fwd_amd/csrc/fa_fwd_inst16.hip",
                  "tiled_exact_attention_fwd_amd/csrc/fa_fwd_inst32.hip",
                  "tiled_exact_attention_fwd_amd/csrc/fa_fwd.hip")
# the instance bench.py times for the headline (bf16, d=128, non-causal)
HEADLINE_KERNEL = "fa::Fwd16P<fa::BF16, 128, false, false>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_d128_n4096_counters.txt")


def kernel_hash():
    """Hash of the kernel sources with comments and whitespace removed, so
    that only a change of code invalidates the stored counter readings."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def upload(words, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(words.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(words).cuda()


class ClockProbe:
    """The shader clock at a point of a stream: fa_clock_probe
    (include/fa_probe.h) counts shader cycles over 20 us of the constant-rate
    real-time counter on 64 CUs, right after the work whose clock it reads
    (the power manager reacts over milliseconds).  mhz() gives the mean and
    range over the CUs of each of the last two probes."""

    WAVES = 64
    TICKS_US = 20

    def __init__(self):
        import torch
        import tiled_exact_attention_fwd_amd as fa
        self.fa = fa
        self.buf = torch.zeros(2 * 2 * self.WAVES, dtype=torch.int64, device="cuda")
        self.tick_hz = self.attribute_khz(10017) * 1e3   # hipDeviceAttributeWallClockRate

    @staticmethod
    def attribute_khz(attr):
        from ctypes import CDLL, byref, c_int
        v = c_int(0)
        if CDLL("libamdhip64.so").hipDeviceGetAttribute(byref(v), attr, 0) != 0 or v.value <= 0:
            raise RuntimeError(f"hipDeviceGetAttribute({attr}) failed")
        return v.value

    def mark(self, i, stream):
        ticks = int(self.TICKS_US * 1e-6 * self.tick_hz)
        st = self.fa.fa_clock_probe(self.buf.data_ptr() + 8 * 2 * self.WAVES * i, ticks, stream)
        if st != self.fa.FA_OK:
            raise RuntimeError(f"fa_clock_probe: {self.fa.fa_strerror(st)}")

    def mhz(self):
        """[(mean, min, max) MHz over the CUs] for the probe before and after."""
        v = self.buf.cpu().tolist()
        res = []
        for i in range(2):
            per = [v[2 * (i * self.WAVES + w)] / (v[2 * (i * self.WAVES + w) + 1] / self.tick_hz) / 1e6
                   for w in range(self.WAVES) if v[2 * (i * self.WAVES + w) + 1] > 0]
            res.append((sum(per) / len(per), min(per), max(per)) if per else None)
        return res


def window_summary(per, probe_mhz):
    """Per-launch durations of the window that follows the bracketed one
    (same launches, an event between consecutive ones), and the rate of the
    shader cycle counter that probes read right before the bracketed
    window's first and right after its last launch (mean over 64 CUs).  The probes run after the load
    has stopped: they read the clock the power manager has set, while inside
    the matrix-core-bound kernel the same counter advances more slowly (the
    chip's fast current limiter), so no fraction of a peak is derived from
    them."""
    out = {"launch_ms": {"first": round(per[0], 5), "max": round(max(per), 5), "min": round(min(per), 5),
                         "mean": round(sum(per) / len(per), 5), "last": round(per[-1], 5),
                         "how": "the same launches right after the bracketed window, an event between each two"}}
    if probe_mhz and all(probe_mhz):
        out["cycle_counter_mhz"] = {"before": round(probe_mhz[0][0], 1), "after": round(probe_mhz[1][0], 1),
                                    "cu_range_after": [round(probe_mhz[1][1], 1), round(probe_mhz[1][2], 1)]}
    return out


def prepare_forward(wl):
    """The workload's seeded inputs uploaded to HBM, and its output buffers."""
    import torch
    import fa_workloads as W
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    q, k, v = (upload(w, wl.dtype) for w in words)
    return q, k, v, torch.empty_like(q), torch.empty(wl.shape[:3], dtype=torch.float32, device=q.device)


def time_workload(wl, causal, steps, warmup, probe=None, tensors=None):
    """Returns dict with ms_per_step (the bracketed window: `steps` launches
    back to back between two events and nothing else on the stream), the
    per-launch durations of a second window of as many launches right after
    it (an event between consecutive launches, so that they tile that
    window's time exactly; the events add about 0.6% to a step), the shader
    clock just before and after the bracketed window (clock probes), and the
    per-launch mean/median/min of a later run of individually timed
    launches."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    q, k, v, o, lse = tensors if tensors is not None else prepare_forward(wl)
    scale = W.scale_for(wl.d)
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    code = fa.dtype_code(q.dtype)
    B, H, N, d = wl.shape
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            B, H, N, d, scale, int(causal), handle, code)

    def step():
        st = fa.fa_fwd(*args)
        if st != fa.FA_OK:
            raise RuntimeError(f"fa_fwd failed: {fa.fa_strerror(st)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # bracketed region: exactly `steps` launches between two events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if probe:
        probe.mark(0, handle)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    if probe:
        probe.mark(1, handle)
    torch.cuda.synchronize()
    bracket_ms = e0.elapsed_time(e1)
    mhz = probe.mhz() if probe else None
    # the same launches again, ev[0] .. ev[steps] splitting the window per launch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    inside = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    # per-launch durations of a later run, each launch alone between two events
    ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev2[2 * i].record(stream)
        step()
        ev2[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev2[2 * i].elapsed_time(ev2[2 * i + 1]) for i in range(steps))
    del q, k, v, o, lse
    return dict(ms_per_step=bracket_ms / steps, inside=inside, sclk_mhz=mhz, launch_mean_ms=sum(per) / len(per),
                launch_median_ms=per[len(per) // 2], launch_min_ms=per[0])


def cold_cache(wl, reps=20):
    """Each launch of the headline workload timed alone after writing a
    512 MiB buffer (more than the 256 MB memory-side cache), so that Q, K and
    V come from HBM."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    q, k, v = (upload(w, wl.dtype) for w in words)
    o = torch.empty_like(q)
    lse = torch.empty(wl.shape[:3], dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    B, H, N, d = wl.shape
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
            W.scale_for(d), 0, stream.cuda_stream, fa.dtype_code(q.dtype))
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
    per = []
    for _ in range(reps):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if fa.fa_fwd(*args) != fa.FA_OK:
            raise RuntimeError("fa_fwd failed")
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    per.sort()
    del q, k, v, o, lse, flush
    return {"median_ms": round(per[len(per) // 2], 5), "min_ms": round(per[0], 5),
            "TFLOP/s": round(wl.flops(False) / (per[len(per) // 2] * 1e-3) / 1e12, 2),
            "how": "each launch timed alone after writing a 512 MiB buffer"}


PROBE_MODES = [("v_exp_f32", 16), ("v_fma_f32", 16), ("v_add_f32", 16), ("v_cvt_pk_bf16_f32 (+xor)", 8),
               ("softmax pair: 2 fma, 2 exp, 1 pack (+xor), 2 add", 4), ("v_mfma_f32_32x32x16_bf16", 4),
               ("MFMA + 1 softmax pair (d = 64 ratio)", 4), ("MFMA + 1/2 softmax pair (d = 128 ratio)", 4)]


def issue_probe(iters=20000):
    """fa_issue_probe (include/fa_probe.h) over every mode: the chip-level
    time per instruction (or per MFMA, or per softmax pair) per SIMD, and the
    ceilings it implies.  The mixes hold no memory traffic, LDS reads or
    barriers: what the VALU and the matrix cores sustain together, two waves
    per SIMD, at the clock the chip holds under that load."""
    import torch
    import tiled_exact_attention_fwd_amd as fa
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    waves, simds = 8 * cus, 4 * cus
    buf = torch.zeros(3 * waves, dtype=torch.int64, device="cuda")
    tick_ns = 1e9 / (ClockProbe.attribute_khz(10017) * 1e3)
    h = torch.cuda.current_stream().cuda_stream
    res = {}
    for mode, (name, n) in enumerate(PROBE_MODES):
        for _ in range(2):      # the first run settles the clock for this mix
            st = fa.fa_issue_probe(mode, iters, buf.data_ptr(), buf.numel(), h)
            if st != fa.FA_OK:
                raise RuntimeError(f"fa_issue_probe: {fa.fa_strerror(st)}")
        torch.cuda.synchronize()
        v = buf.view(-1, 3).cpu()
        wall_ns = (int(v[:, 2].max()) - int(v[:, 1].min())) * tick_ns
        res[name] = wall_ns * simds / (waves * iters * n)
    mfma = res["v_mfma_f32_32x32x16_bf16"]
    flop = 2 * 32 * 32 * 16
    out = {"ns_per_instruction_per_simd": {k: round(v_, 3) for k, v_ in res.items()},
           "mfma_TFLOP/s": round(flop / mfma * simds / 1e3, 1),
           "ceiling_TFLOP/s": {
               "d64": round(flop / res["MFMA + 1 softmax pair (d = 64 ratio)"] * simds / 1e3, 1),
               "d128": round(flop / res["MFMA + 1/2 softmax pair (d = 128 ratio)"] * simds / 1e3, 1)},
           # the softmax alone: a pair instruction is 2 scores on each of 64 lanes, a score 4 d FLOPs
           "softmax_only_TFLOP/s": {
               "d64": round(128 * 4 * 64 / res["softmax pair: 2 fma, 2 exp, 1 pack (+xor), 2 add"] * simds / 1e3, 1),
               "d128": round(128 * 4 * 128 / res["softmax pair: 2 fma, 2 exp, 1 pack (+xor), 2 add"] * simds / 1e3,
                             1)},
           "cus": cus}
    return out


def backward_flops(wl, causal):
    """10 B H N^2 d: the five N x N x d products of the backward (recomputed
    S, dP, dV, dK, dQ), 2.5 times the forward's convention, halved causal.
    The kernels run seven (S and dP in each of the two kernels); the extra
    work is not counted."""
    return 2.5 * wl.flops(causal)


def prepare_backward(wl, causal):
    """Inputs of the backward on a workload: Q, K, V, the seeded dO, and the
    forward's O and LSE (one forward launch); gradient and work buffers."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    q, k, v = (upload(w, wl.dtype) for w in words)
    do = upload(W.encode(W.draw_dout(wl.shape, W.default_seed()), wl.dtype), wl.dtype)
    o, lse = fa.attention(q, k, v, causal=causal, scale=W.scale_for(wl.d))
    return q, k, v, do, o, lse, torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(lse)


def time_backward(wl, causal, steps, warmup, tensors=None):
    """fa_bwd (dQ and D kernel, then dK/dV kernel) on a workload; the
    forward runs once beforehand for O and LSE.  Returns ms per step."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    q, k, v, do, o, lse, dq, dk, dv, delta = tensors if tensors is not None else prepare_backward(wl, causal)
    scale = W.scale_for(wl.d)
    stream = torch.cuda.current_stream()
    B, H, N, d = wl.shape
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale, int(causal),
            stream.cuda_stream, fa.dtype_code(q.dtype))

    def step():
        st = fa.fa_bwd(*args)
        if st != fa.FA_OK:
            raise RuntimeError(f"fa_bwd failed: {fa.fa_strerror(st)}")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del q, k, v, do, o, lse, dq, dk, dv, delta
    return ms


BACKWARD_CASES = [("non_causal", "C2b", False), ("causal", "C3", True)]


def backward_summary(steps, warmup, more=False, prepared=None):
    import fa_workloads as W
    out = {}
    cases = list(BACKWARD_CASES)
    if more:   # the ragged d = 64 workload, and fp16 at the headline shape
        cases += [("C4_non_causal", "C4", False), ("C4_causal", "C4", True), ("C2_fp16_non_causal", "C2", False)]
    for key, name, causal in cases:
        wl = W.WORKLOADS[name]
        ms = time_backward(wl, causal, steps, warmup, (prepared or {}).get(key))
        tf = backward_flops(wl, causal) / (ms * 1e-3) / 1e12
        out[key] = {"ms_per_step": round(ms, 5), "value": round(tf, 2), "frac": round(tf / PEAK_TFLOPS["bf16"], 4)}
    out["unit"] = "TFLOP/s"
    out["workload"] = ("backward with recomputation (dQ, dK, dV from O, LSE, dO), B=4 H=16 N=4096 d=128 bf16; "
                       "causal with 1% of key rows x8; 10 B H N^2 d FLOPs, halved causal")
    return out


def split_kv(steps, warmup):
    """Split-KV forward against the plain launch on few-head long sequences:
    bf16, d = 128, non-causal and causal."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    rows = []
    for (B, H, N, causal) in ((1, 1, 32768, 0), (1, 2, 16384, 0), (1, 4, 8192, 0), (1, 8, 4096, 0),
                              (1, 1, 32768, 1), (1, 4, 32768, 1), (1, 8, 16384, 1), (1, 32, 32768, 1)):
        shape = (B, H, N, 128)
        words = W.make_words(shape, "bf16", "normal", W.default_seed())
        q, k, v = (upload(w, "bf16") for w in words)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        op = torch.empty((16, B, H, N, 128), dtype=torch.float32, device=q.device)
        lp = torch.empty((16, B, H, N), dtype=torch.float32, device=q.device)
        handle = torch.cuda.current_stream().cuda_stream
        scale = W.scale_for(128)
        flops = 4.0 * B * H * N * N * 128 / (2 if causal else 1)
        tq = 128 if causal else 256
        res = {"B": B, "H": H, "N": N, "causal": bool(causal), "query_tiles": B * H * ((N + tq - 1) // tq)}
        for splits in (0, 2, 4, 8, 16):
            def step():
                if splits == 0:
                    st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                                   128, scale, causal, handle, fa.FA_DTYPE_BF16)
                else:
                    st = fa.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         op.data_ptr(), lp.data_ptr(), B, H, N, 128, scale, causal, splits, handle,
                                         fa.FA_DTYPE_BF16)
                if st != fa.FA_OK:
                    raise RuntimeError(fa.fa_strerror(st))
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            res["plain" if splits == 0 else f"split{splits}"] = {"ms": round(ms, 4),
                                                                  "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
        print(json.dumps(res), flush=True)
        del q, k, v, o, lse, op, lp


def all_configs(steps, warmup):
    """Every named workload (C1-C5, each mask setting): forward time and
    TFLOP/s with its fraction of the matching dense MFMA peak, the issue
    ceiling of its head dimension (the matrix work and the softmax of the key
    loop co-issued, from the issue-rate probe, measured first) and its
    fraction of it, and the backward's time and TFLOP/s (10 B H N^2 d, halved
    causal).  One JSON line per workload."""
    import fa_workloads as W
    probe = issue_probe()
    print(json.dumps({"issue_probe": probe}), flush=True)
    for name, wl in W.WORKLOADS.items():
        for causal in wl.causal:
            r = time_workload(wl, causal, steps, warmup)
            f = wl.flops(causal)
            tf = f / (r["launch_mean_ms"] * 1e-3) / 1e12
            row = {"workload": name, "shape": list(wl.shape), "dtype": wl.dtype, "values": wl.values,
                   "causal": causal, "fwd_us": round(r["launch_mean_ms"] * 1e3, 1), "fwd_TFLOP/s": round(tf, 1),
                   "fwd_frac": round(tf / PEAK_TFLOPS[wl.dtype], 4),
                   "alu_peak": probe["ceiling_TFLOP/s"][f"d{wl.d}"] if wl.dtype != "f32" else None,
                   "alu_frac": round(tf / probe["ceiling_TFLOP/s"][f"d{wl.d}"], 4) if wl.dtype != "f32" else None,
                   "hbm_min_GB/s": round((4 * wl.B * wl.H * wl.N * wl.d * (4 if wl.dtype == "f32" else 2)
                                          + 4 * wl.B * wl.H * wl.N) / (r["launch_mean_ms"] * 1e-3) / 1e9, 1)}
            ms = time_backward(wl, causal, max(5, steps // 4), max(3, warmup // 4))
            bt = backward_flops(wl, causal) / (ms * 1e-3) / 1e12
            row.update({"bwd_us": round(ms * 1e3, 1), "bwd_TFLOP/s": round(bt, 1),
                        "bwd_frac": round(bt / PEAK_TFLOPS[wl.dtype], 4)})
            print(json.dumps(row), flush=True)


def cpu_baseline(seconds):
    """The float64 oracle on whole heads of the headline workload -- the same
    16-bit words the GPU receives, decoded exactly -- head by head until about
    `seconds` of CPU work; returns the oracle's TFLOP/s equivalent."""
    import fa_workloads as W
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    wl = W.WORKLOADS["C2b"]
    B, H, N, d = wl.shape
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    scale = W.scale_for(d)
    heads, t_total = 0, 0.0
    while heads < B * H and (t_total < seconds or heads == 0):
        b, h = divmod(heads, H)
        q, k, v = (W.decode64(w[b:b + 1, h:h + 1], wl.dtype) for w in words)
        t = time.perf_counter()
        oracle.attention_ref(q, k, v, scale, False)
        t_total += time.perf_counter() - t
        heads += 1
    flops = 4.0 * N * N * d * heads
    return dict(value=flops / t_total / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"the first {heads} of the {B * H} heads of the headline workload (the same bf16 words "
                       f"the GPU reads), N={N}, d={d}, non-causal, float64 with S and P materialised, "
                       f"{t_total:.1f} s",
                seconds=t_total, host=host_cpu())


def host_cpu():
    """The host's CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"model": model, "usable_cores": usable}


def read_summary(path):
    """`key: value` lines of a profile summary (other lines ignored)."""
    out = {}
    try:
        with open(path) as f:
            for ln in f:
                if ":" in ln and not ln.startswith((" ", "#", "|")):
                    k, v = ln.split(":", 1)
                    out[k.strip()] = v.strip()
    except OSError:
        pass
    return out


def traffic_for_kernel():
    """HBM bytes per launch of the C2b kernel from the committed rocprofv3
    counter summary, or None when the kernel sources changed since the
    counters were taken."""
    t = read_summary(TRAFFIC_FILE)
    if t.get("kernel_hash") != kernel_hash() or "hbm_bytes_per_launch" not in t:
        return None
    return int(t["hbm_bytes_per_launch"])


def summarize(kind, paths):
    """Text summary of rocprofv3 output for profiles/.
    kind 'trace': a --kernel-trace --stats directory (csv output).
    kind 'counters': the FETCH_SIZE and WRITE_SIZE --pmc directories (csv),
    scaled by what the same counters read for the copy kernel of known size
    that --profile-run launches first."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not files:
            raise SystemExit(f"no {pattern} under {d}")
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    if kind == "trace":
        # 'trace DIR [K [S]]': the K dispatches of a kernel after the first S
        # (default: its last K) -- for the headline kernel, S = 200 and K = 100
        # are the launches the bench times one by one (its launch_ms)
        count = int(paths[1]) if len(paths) > 1 else 100
        skip = int(paths[2]) if len(paths) > 2 else None
        durs = {}
        for r in sorted(rows(paths[0], "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
            durs.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        label = f"last {count}" if skip is None else f"dispatches {skip + 1}-{skip + count}"
        print(f"| kernel | calls | average us | min us | max us | average of the {label} us |")
        print("|---|---|---|---|---|---|")
        for r in rows(paths[0], "*kernel_stats.csv"):
            name = r["Name"]
            if "fa::" not in name:
                continue
            d = durs.get(name, [])
            sel = d[-count:] if skip is None else d[skip:skip + count]
            avg = f"{sum(sel) / len(sel):.1f}" if sel else "-"
            print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {avg} |")
        return
    if kind == "pmc":
        # 'pmc DIR...': rocprofv3 --pmc runs of --profile-run, each with its own
        # counters; per forward kernel the median over its dispatches, and
        # the ratios that locate its cycles
        vals = {}
        agent = {"Num_Shader_Banks": 32, "Num_Xcc": 8, "Simd_Count": 1024}
        for r in rows(paths[0], "*agent_info.csv"):
            if r.get("Agent_Type") == "GPU":
                agent = {k: int(r[k]) for k in agent}
        print(f"agent: {agent}")
        print()
        for d in paths:
            for r in rows(d, "*counter_collection.csv"):
                if "fa::" not in r["Kernel_Name"]:
                    continue
                vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
        for name, cs in sorted(vals.items()):
            med = {c: statistics.median(v) for c, v in cs.items()}
            print(f"## {name}")
            print()
            print("| counter | dispatches | median per dispatch |")
            print("|---|---|---|")
            for c in sorted(med):
                print(f"| {c} | {len(cs[c])} | {med[c]:.6g} |")
            print()
            ratio = []
            # rocprofv3 sums each counter over its instances: SQ_CYCLES over the
            # shader engines, GRBM_GUI_ACTIVE over the XCDs, the busy cycles
            # over the SIMDs (the agent's Num_Shader_Banks, Num_Xcc, Simd_Count)
            ses, xccs, simds = agent["Num_Shader_Banks"], agent["Num_Xcc"], agent["Simd_Count"]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "SQ_CYCLES" in med:
                ratio.append(("MFMA busy fraction of the dispatch's cycles (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / "
                              "(SQ_CYCLES / shader engines))",
                              med["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (med["SQ_CYCLES"] / ses)))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
                ratio.append(("the same against GRBM_GUI_ACTIVE / XCDs",
                              med["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / (med["GRBM_GUI_ACTIVE"] / xccs)))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "SQ_INSTS_MFMA" in med:
                ratio.append(("MFMA busy cycles per MFMA instruction",
                              med["SQ_VALU_MFMA_BUSY_CYCLES"] / med["SQ_INSTS_MFMA"]))
            if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
                ratio.append(("matrix FLOPs (MOPS_BF16 x 512)", med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512))
            if "SQ_INSTS_MFMA" in med:
                for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_SMEM", "SQ_INSTS_VALU_TRANS_F32",
                          "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_ADD_F32", "SQ_INSTS_VALU_CVT", "SQ_INSTS_VMEM"):
                    if c in med:
                        ratio.append((f"{c} per MFMA", med[c] / med["SQ_INSTS_MFMA"]))
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in med and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
                ratio.append(("cycles with a VALU issue under a busy MFMA / MFMA busy cycles",
                              med["SQ_VALU_MFMA_COEXEC_CYCLES"] / med["SQ_VALU_MFMA_BUSY_CYCLES"]))
            if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
                ratio.append(("LDS bank-conflict cycles / LDS active cycles",
                              med["SQ_LDS_BANK_CONFLICT"] / max(med["SQ_LDS_IDX_ACTIVE"], 1)))
            if "SQ_ACTIVE_INST_VALU" in med and "SQ_CYCLES" in med:
                ratio.append(("VALU-active fraction of a SIMD's cycles (SQ_ACTIVE_INST_VALU x 4 / SIMDs / "
                              "(SQ_CYCLES / shader engines))",
                              med["SQ_ACTIVE_INST_VALU"] * 4 / simds / (med["SQ_CYCLES"] / ses)))
            if "SQ_WAIT_INST_ANY" in med and "SQ_WAVE_CYCLES" in med:
                ratio.append(("wave cycles waiting for an instruction's issue / wave cycles",
                              med["SQ_WAIT_INST_ANY"] / med["SQ_WAVE_CYCLES"]))
            if "SQ_ACTIVE_INST_VALU" in med and "SQ_WAVE_CYCLES" in med:
                ratio.append(("wave cycles on VALU instructions / wave cycles",
                              med["SQ_ACTIVE_INST_VALU"] / med["SQ_WAVE_CYCLES"]))
            if ratio:
                print("| derived | value |")
                print("|---|---|")
                for k_, v_ in ratio:
                    print(f"| {k_} | {v_:.4g} |")
                print()
        return
    if kind == "l2":
        hits, misses = {}, {}
        for r in rows(paths[0], "*counter_collection.csv"):
            dst = hits if r["Counter_Name"] == "TCC_HIT_sum" else misses
            dst.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        print("| kernel | dispatches | L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)) |")
        print("|---|---|---|")
        for name in sorted(hits):
            if "fa::" not in name:
                continue
            h, m = statistics.median(hits[name]), statistics.median(misses.get(name, [0.0]))
            print(f"| {name} | {len(hits[name])} | {h / (h + m):.3f} |")
        return
    per = {}
    for d in paths:
        for r in rows(d, "*counter_collection.csv"):
            key = (r["Kernel_Name"], r["Counter_Name"])
            per.setdefault(key, []).append(float(r["Counter_Value"]))
    copy_bytes = 64 * (1 << 20) * 4
    fetch_copy = statistics.median(v for (k, c), vals in per.items() if "copyBuffer" in k and c == "FETCH_SIZE"
                                   for v in vals)
    write_copy = statistics.median(v for (k, c), vals in per.items() if "copyBuffer" in k and c == "WRITE_SIZE"
                                   for v in vals)
    f_fetch = copy_bytes / (fetch_copy * 1024)
    f_write = copy_bytes / (write_copy * 1024)
    print(f"kernel_hash: {kernel_hash()}")
    print(f"copy_fetch_factor: {f_fetch:.4f}")
    print(f"copy_write_factor: {f_write:.4f}")
    total = 0.0
    for (k, c), vals in per.items():
        if HEADLINE_KERNEL in k:
            total += statistics.median(vals) * 1024 * (f_fetch if c == "FETCH_SIZE" else f_write)
    print(f"hbm_bytes_per_launch: {int(round(total))}")
    print()
    print("| kernel | counter | dispatches | median raw | scaled |")
    print("|---|---|---|---|---|")
    for (k, c), vals in sorted(per.items()):
        if "fa::" not in k:
            continue
        scale = f_fetch if c == "FETCH_SIZE" else f_write
        print(f"| {k} | {c} | {len(vals)} | {statistics.median(vals):.0f} KiB | "
              f"{statistics.median(vals) * 1024 * scale / (1 << 20):.2f} MiB scaled |")


def copy_calibration():
    """Copy kernel of known size: what FETCH_SIZE / WRITE_SIZE read for it
    scales the counters of the other kernels."""
    import torch
    src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy kernel: {src.numel() * 4} bytes read, {dst.numel() * 4} bytes written", flush=True)


def profile_run():
    """Copy kernel of known size (counter calibration), then the forward."""
    import fa_workloads as W
    copy_calibration()
    for name, causal in (("C2b", False), ("C3", True)):
        r = time_workload(W.WORKLOADS[name], causal, 3, 1)
        print(f"{name} causal={causal}: {r}", flush=True)


def standard_baseline(steps, warmup):
    """The standard forward (S and P in HBM) on the C2b workload."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    copy_calibration()
    wl = W.WORKLOADS["C2b"]
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    q, k, v = (upload(w, wl.dtype) for w in words)
    B, H, N, d = wl.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    sm = torch.empty((B, H, N, N), dtype=q.dtype, device=q.device)
    pm = torch.empty_like(sm)
    handle = torch.cuda.current_stream().cuda_stream

    def step():
        st = fa.fa_standard_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                sm.data_ptr(), pm.data_ptr(), B, H, N, d, W.scale_for(d), 0, handle,
                                fa.FA_DTYPE_BF16)
        if st != fa.FA_OK:
            raise RuntimeError(f"fa_standard_fwd: {fa.fa_strerror(st)}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"standard_forward": "S and P materialised", "workload": "B=4 H=16 N=4096 d=128 bf16 non-causal",
                      "ms_per_step": round(ms, 4), "TFLOP/s": round(wl.flops(False) / (ms * 1e-3) / 1e12, 2),
                      "S_and_P_bytes": 2 * B * H * N * N * 2}), flush=True)


SWEEP_TILES = [(64, 32), (64, 64), (64, 128), (128, 32), (128, 64), (128, 128),
               (256, 32), (256, 64), (256, 128)]


def sweep_kernel_key(tq, tk):
    """Mangled-name fragment of the plain per-tile kernel of one sweep shape."""
    waves = 0 if (tq, tk) == (256, 64) else tq // 32
    return f"Fwd16INS_4BF16ELi128ELb0ELb0ELb0ELi{waves}ELi{tk}E"


def tile_sweep(steps, warmup):
    """Tile-size sweep at the C2b shape: TFLOP/s and kernel resources per shape."""
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    from tiled_exact_attention_fwd_amd import codeobj
    wl = W.WORKLOADS["C2b"]
    words = W.make_words(wl.shape, wl.dtype, wl.values, W.default_seed())
    q, k, v = (upload(w, wl.dtype) for w in words)
    o = torch.empty_like(q)
    lse = torch.empty(wl.shape[:3], dtype=torch.float32, device=q.device)
    B, H, N, d = wl.shape
    handle = torch.cuda.current_stream().cuda_stream
    res = codeobj.kernel_resources(fa.LIB_PATH)
    print(f"| tile (query rows x keys) | TFLOP/s | % of peak | VGPR (arch+acc) | spilled VGPRs | "
          f"LDS bytes | waves per SIMD | working set, 16-bit tiles (bytes) |")
    print("|---|---|---|---|---|---|---|---|")
    for tq, tk in SWEEP_TILES:
        def launch():
            st = fa.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, N, d, W.scale_for(d), 0, handle, fa.FA_DTYPE_BF16, tile_q=tq, tile_k=tk)
            if st != fa.FA_OK:
                raise RuntimeError(f"fa_fwd_ex {tq}x{tk}: {fa.fa_strerror(st)}")
        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            launch()
        e1.record()
        torch.cuda.synchronize()
        tf = wl.flops(False) / (e0.elapsed_time(e1) / steps * 1e-3) / 1e12
        key = sweep_kernel_key(tq, tk)
        r = next(v_ for n_, v_ in res.items() if key in n_)
        waves = tq // 32
        # waves per SIMD: the launch bound (2), the register file (512 per
        # lane), and the LDS (160 KiB per CU, shared by the workgroups)
        regs = -(-r["vgpr"] // 8) * 8
        occ = min(2, 512 // regs, (160 * 1024 // r["lds"]) * waves / 4)
        ws = (2 * tq * d + 2 * tk * d + tq * tk) * 2
        print(f"| {tq} x {tk} | {tf:.1f} | {100 * tf / PEAK_TFLOPS['bf16']:.1f}% | {r['vgpr']} | "
              f"{r['vgpr_spill']} | {r['lds']} | {occ:g} | {ws} |", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the chip settles its clock under this load after a few tens of launches
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="tile-size sweep table")
    ap.add_argument("--standard", action="store_true", help="time the standard (materialising) forward")
    ap.add_argument("--backward", action="store_true", help="time only the backward pass (fa_bwd)")
    ap.add_argument("--split", action="store_true", help="split-KV forward against the plain one, few heads")
    ap.add_argument("--configs", action="store_true", help="forward and backward on every named workload")
    ap.add_argument("--issue-probe", action="store_true", help="issue rates of the key loop's instruction mixes")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="print a profiles/ summary of rocprofv3 csv output: "
                         "'trace DIR [COUNT [SKIP]]', 'counters FETCH_DIR WRITE_DIR', 'l2 DIR' or 'pmc DIR...'")
    a = ap.parse_args()
    if a.summarize:
        summarize(a.summarize[0], a.summarize[1:])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(a.gpus, world)}): the forward "
              "kernel runs on a single MI355X; multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import fa_workloads as W
    import tiled_exact_attention_fwd_amd as fa
    fa.lib()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if a.profile_run:
        profile_run()
        return
    if a.sweep:
        tile_sweep(a.steps, a.warmup)
        return
    if a.standard:
        standard_baseline(a.steps, a.warmup)
        return
    if a.split:
        split_kv(a.steps, a.warmup)
        return
    if a.configs:
        all_configs(a.steps, a.warmup)
        return
    if a.issue_probe:
        print(json.dumps({"issue_probe": issue_probe()}), flush=True)
        return
    if a.backward:
        copy_calibration()
        print(json.dumps({"backward": backward_summary(a.steps, a.warmup, more=True)}), flush=True)
        return

    # Every input of the line's measurements is made resident in HBM first;
    # the measurements then run back to back, with no idle time between them,
    # in this order: the backward, the causal launch, the headline launch.
    # (The power manager of a GPU that was idle reacts to a rise in load with
    # a clock dip that lasts a few tens of milliseconds -- the first launches
    # run fast, the next ones up to ~20% slow, then steady -- and repeats it
    # after every idle stretch; here the secondary measurements take it.)
    # Every window's per-launch durations and average shader clock are in the
    # line, so each figure can be checked against them.
    probe = ClockProbe()
    wc, wl = W.WORKLOADS["C3"], W.WORKLOADS["C2b"]
    fw_causal, fw_head = prepare_forward(wc), prepare_forward(wl)
    bw_inputs = {key: prepare_backward(W.WORKLOADS[name], causal) for key, name, causal in BACKWARD_CASES}
    torch.cuda.synchronize()

    bwd = backward_summary(max(10, a.steps // 4), max(5, a.warmup // 4), prepared=bw_inputs)
    del bw_inputs

    rc = time_workload(wc, True, a.steps, a.warmup, probe, fw_causal)
    fc = wc.flops(True)
    causal_value = fc / (rc["ms_per_step"] * 1e-3) / 1e12

    r = time_workload(wl, False, a.steps, a.warmup, probe, fw_head)
    flops = wl.flops(False)
    value = flops / (r["ms_per_step"] * 1e-3) / 1e12
    # the headline kernel's average launch duration over the timed region:
    # its only work is that kernel's launches
    achieved = value
    cold = cold_cache(wl)
    traffic = traffic_for_kernel()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention forward B=4 H=16 N=4096 d=128 bf16 non-causal, "
                               "Q/K/V i.i.d. N(0,1), scale 1/sqrt(128)",
                   "B": 4, "H": 16, "N": 4096, "d": 128, "causal": False,
                   "tile": list(fa.fa_fwd_tile_shape(fa.FA_DTYPE_BF16, 128, 0)[1:])},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic},
        "window": window_summary(r["inside"], r["sclk_mhz"]),
        "order": ("inputs uploaded first; then back to back: backward, causal, headline (each: its warmup "
                  "launches, then its timed launches)"),
        "causal": {"workload": "same shape, causal, 1% of key rows x8",
                   "value": round(causal_value, 2), "unit": "TFLOP/s",
                   "ms_per_step": round(rc["ms_per_step"], 5),
                   "frac": round(causal_value / PEAK_TFLOPS["bf16"], 4),
                   "window": window_summary(rc["inside"], rc["sclk_mhz"])},
        "backward": bwd,
        "cold_cache": cold,
        "settled_launch_ms": {"mean": round(r["launch_mean_ms"], 5), "median": round(r["launch_median_ms"], 5),
                              "min": round(r["launch_min_ms"], 5),
                              "how": "a later run of the same launches, each alone between two events"},
        "hbm_min_gbs": round((4 * wl.B * wl.H * wl.N * wl.d * 2 + 4 * wl.B * wl.H * wl.N)
                             / (r["ms_per_step"] * 1e-3) / 1e9, 1),
        "kernel_hash": kernel_hash(),
    }
    if not a.no_cpu_baseline:
        cb = cpu_baseline(a.cpu_seconds)
        out["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v)
                               for k, v in cb.items() if k != "seconds"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
