"""Benchmark of the FP8 block-scaled GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]

A step is one pass over the dense LLM-layer workload: the 15 GEMMs
M in {64, 128, 4096} x (N, K) in {(2112,7168), (24576,1536), (7168,16384),
(4096,7168), (7168,2048)}, inputs quantized once (device-side fp32 draws, the
library's own cast kernels) and resident in HBM before timing.  ``value`` is
whole-step TFLOPS (2*M*N*K summed over the step / wall time of K steps).

The JSON line also carries:
* ``roofline``: the dominant kernel (the tile/split instance that takes most of
  the step), algorithmic FLOPs per launch / its average launch time, against
  the 5.0 PFLOP/s dense FP8 MFMA peak (2.4 GHz), and against 256 CUs x 8192
  FLOP/clock at the clock the committed counter pass measured for it.  The launch time is measured inside the
  timed steps with HIP events on the launch stream, one pair around each run of
  consecutive launches of that instance (event time / launches).  Events
  between launches cost GPU time, so the timed steps carry no others;
* ``per_shape``: ``us_in_step`` from separate untimed steps with an event pair
  around every launch, and cold-cache times (operands evicted before each run).
  Each shape also gets its roofline ceiling, min(FP8 peak, FLOPs / minimal
  bytes x HBM peak), and the cold rate as a percentage of that ceiling (the
  M <= 128 shapes are bound by streaming B, not by the MFMA).  The M <= 128
  shapes also get ``us_cold_pipelined``: back-to-back launches over distinct
  operand copies (> 512 MB in all, so every launch still reads HBM), replayed
  from a HIP graph, which removes the per-launch event overhead of a single
  short launch;
* ``event_floor_us``: the event time of a one-element fill kernel measured like
  the cold times, the least an event pair around one launch reads here;
* ``cpu_baseline``: the CPU oracle on the whole dense workload (every GEMM at
  full size), on group samples of the MoE workloads and a row sample of the
  cast, with the CPU model, BLAS library and thread count;
* ``extras``: the MoE workloads (contiguous G=8, masked G=16 with its decode
  variant, Zipf contiguous G=256 with power-of-two scales), each with the same
  ceiling, and the per-token cast of a bf16 [32768, 7168] activation in GB/s.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E


def min_bytes(rows, n, k, groups=1):
    """Bytes a GEMM must move at least: the useful A rows, every group's B, both
    scale arrays and D, each once (fp32 scale words)."""
    kb = k // 128
    return rows * k + groups * n * k + 4 * rows * kb + 4 * groups * ((n + 127) // 128) * kb + 2 * rows * n


def ceiling_tflops(flops, nbytes):
    """Roofline ceiling of one GEMM: the smaller of the FP8 MFMA peak and its
    arithmetic intensity times the HBM peak."""
    return min(FP8_PEAK_TFLOPS, flops / nbytes * HBM_PEAK_GBS / 1e3)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def mn_major(rows, kblocks, dev, groups=None):
    """Scale buffer for A in the MN-major ("transposed") layout the GEMM reads
    best: element (row, kb) at kb * rows + row."""
    if groups is None:
        return torch.empty((kblocks, rows), dtype=torch.float32, device=dev).t()
    return torch.empty((groups, kblocks, rows), dtype=torch.float32, device=dev).transpose(1, 2)


def make_dense(dg, m, n, k, seed, dev):
    a32 = synth.draw_activation_device(m, k, seed, dev)
    b32 = synth.draw_weight_device(n, k, seed, 0, dev)
    qa, sa = dg.per_token_cast_fp8(a32, sf=mn_major(m, k // 128, dev))
    qb, sb = dg.per_block_cast_fp8(b32)
    del a32, b32
    d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    return (qa, sa), (qb, sb), d


def packed_mn_major(dg, sf, dev, groups=None):
    """Packed UE8M0 words of power-of-two fp32 scales [..., rows, kblocks], in the
    MN-major layout for A: word (row, w) at w * rows + row."""
    rows, kb = sf.shape[-2], sf.shape[-1]
    words = (kb + 3) // 4
    if groups is None:
        out = torch.empty((words, rows), dtype=torch.int32, device=dev).t()
    else:
        out = torch.empty((groups, words, rows), dtype=torch.int32, device=dev).transpose(1, 2)
    return dg.pack_ue8m0(sf, out=out)


class Flusher:
    """Reads a 1 GiB buffer so that cold-cache timings do not see operands left in
    the 256 MB Infinity Cache (MALL) or the L2s.  It reads rather than writes: a
    write flush leaves the MALL full of dirty lines whose write-back would then
    be charged to the timed kernel."""

    def __init__(self, dev, nbytes=1 << 30):
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        torch.sum(self.buf, dim=0, out=self.sink)


def event_time_ms(fn, reps, flush=None, warmup=5):
    """Median HIP-event time of fn over reps runs, each after the cache flush.
    The untimed warm-up runs (same flush) let the clocks settle first: the
    first launches of a workload in a process run up to 10% slower."""
    for _ in range(warmup):
        if flush:
            flush()
        fn()
    times = []
    for _ in range(reps):
        if flush:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    return float(np.median(times))


def event_floor_us(dev, reps=20):
    """Event time of the smallest kernel (a one-element fill), measured the way
    the cold per-shape times are (after the cache-evicting read, so the host
    has queued the kernel before the GPU reaches it): the least an event pair
    around one launch reads here."""
    x = torch.empty(1, dtype=torch.float32, device=dev)
    flush = Flusher(dev)
    us = event_time_ms(lambda: x.zero_(), reps, flush) * 1e3
    del flush
    return us


def pipelined_cold_us(dg, a, b, d, min_bytes_total=600 << 20, reps=5):
    """Per-launch time of R back-to-back launches of one GEMM, each on its own
    copy of the operands, R copies spanning more than the 256 MB last-level
    cache (and the flush) so that every launch reads cold operands.  The R
    launches are captured once as a HIP graph and replayed, so host-side call
    overhead does not enter the time."""
    nbytes = a[0].numel() + b[0].numel() + 4 * (a[1].numel() + b[1].numel())
    r = max(4, -(-min_bytes_total // nbytes))
    copies = [((a[0].clone(), a[1].clone()), (b[0].clone(), b[1].clone()), torch.empty_like(d)) for _ in range(r)]
    m, n, k = a[0].shape[0], b[0].shape[0], a[0].shape[1]
    ws = torch.zeros(max(dg.workspace_size(m, n, k), 16), dtype=torch.uint8, device=d.device)

    def run():
        for aa, bb, dd in copies:
            dg.fp8_gemm_nt(aa, bb, dd, workspace=ws)
    run()                                   # outside the capture: first-call set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    flush = Flusher(a[0].device)
    ms = event_time_ms(graph.replay, reps, flush, warmup=2)
    del copies, flush, graph, ws
    torch.cuda.empty_cache()
    return ms * 1e3 / r


def bench_extras(dg, dev, reps):
    out = {}
    flush = Flusher(dev)
    traffic = counted_traffic()
    # --- the small parity-sized problem (128 x 256 x 512): launch latency
    log("extras: dense 128x256x512")
    a0, b0, d0 = make_dense(dg, 128, 256, 512, synth.seed_for(0, 0), dev)
    ms0 = event_time_ms(lambda: dg.fp8_gemm_nt(a0, b0, d0), reps, flush)
    stream0 = torch.cuda.Stream()
    stream0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream0):
        dg.fp8_gemm_nt(a0, b0, d0)
    torch.cuda.synchronize()
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g0, stream=stream0):
        for _ in range(100):
            dg.fp8_gemm_nt(a0, b0, d0)
    g0.replay()
    torch.cuda.synchronize()
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    g0.replay()
    e0.record()
    torch.cuda.synchronize()
    out["dense_128x256x512"] = {"us_cold": ms0 * 1e3, "us_back_to_back_graph": s0.elapsed_time(e0) * 1e3 / 100,
                                "gflop": 2.0 * 128 * 256 * 512 / 1e9}
    del g0, a0, b0, d0
    # --- contiguous G=8 (prefill) and masked G=16 (decode)
    for idx, (n, k) in enumerate(synth.GROUPED_NK):
        counts, m_indices = synth.config2_routing(idx)
        seed = synth.seed_for(2, idx)
        m_total = m_indices.size
        valid = torch.as_tensor(np.nonzero(m_indices >= 0)[0], device=dev)
        a32 = torch.zeros((m_total, k), dtype=torch.float32, device=dev)
        a32[valid] = synth.draw_activation_device(int(valid.numel()), k, seed, dev)
        qa, sa = dg.per_token_cast_fp8(a32, sf=mn_major(m_total, k // 128, dev))
        del a32
        qb = torch.empty((8, n, k), dtype=torch.float8_e4m3fn, device=dev)
        sb = torch.empty((8, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
        for g in range(8):
            dg.per_block_cast_fp8(synth.draw_weight_device(n, k, seed, g, dev), q=qb[g], sf=sb[g])
        d = torch.empty((m_total, n), dtype=torch.bfloat16, device=dev)
        mi = torch.from_numpy(m_indices).to(dev)
        log(f"extras: contiguous G=8 {n}x{k}")
        ms = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((qa, sa), (qb, sb), d, mi), reps, flush)
        useful = 2.0 * int(counts.sum()) * n * k
        ceil = ceiling_tflops(useful, min_bytes(int(counts.sum()), n, k, 8))
        out[f"contiguous_G8_{n}x{k}"] = {
            "us": ms * 1e3, "tflops_useful": useful / ms / 1e9, "tflops_padded": 2.0 * m_total * n * k / ms / 1e9,
            "pct_fp8_peak": 100 * useful / ms / 1e9 / FP8_PEAK_TFLOPS, "m_total": m_total,
            "ceiling_tflops": ceil, "pct_of_ceiling": 100 * useful / ms / 1e9 / ceil,
            "hbm_gbs_counted": counted_gbs(traffic, f"contiguous_G8_{n}x{k}", ms * 1e3)}
        del qa, sa, qb, sb, d

        masked_m = synth.config3_masked_m(idx)
        seed = synth.seed_for(3, idx)
        a32 = synth.draw_activation_device(16 * 256, k, seed, dev).view(16, 256, k)
        qa = torch.empty((16, 256, k), dtype=torch.float8_e4m3fn, device=dev)
        sa = mn_major(256, k // 128, dev, groups=16)
        for g in range(16):
            dg.per_token_cast_fp8(a32[g], q=qa[g], sf=sa[g])
        del a32
        qb = torch.empty((16, n, k), dtype=torch.float8_e4m3fn, device=dev)
        sb = torch.empty((16, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
        for g in range(16):
            dg.per_block_cast_fp8(synth.draw_weight_device(n, k, seed, g, dev), q=qb[g], sf=sb[g])
        d = torch.empty((16, 256, n), dtype=torch.bfloat16, device=dev)
        mm = torch.from_numpy(masked_m).to(dev)
        log(f"extras: masked G=16 {n}x{k}")
        ms = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_masked((qa, sa), (qb, sb), d, mm, 128), reps, flush)
        useful = 2.0 * int(masked_m.sum()) * n * k
        b_bytes = 16 * n * k
        ceil = ceiling_tflops(useful, min_bytes(int(masked_m.sum()), n, k, 16))
        out[f"masked_G16_{n}x{k}"] = {
            "us": ms * 1e3, "tflops_useful": useful / ms / 1e9, "pct_fp8_peak": 100 * useful / ms / 1e9 / FP8_PEAK_TFLOPS,
            "b_read_gbs": b_bytes / ms / 1e6, "ceiling_tflops": ceil, "pct_of_ceiling": 100 * useful / ms / 1e9 / ceil,
            "hbm_gbs_counted": counted_gbs(traffic, f"masked_G16_{n}x{k}", ms * 1e3)}
        # decode shape on the same operands: 0..32 rows per group, run on the
        # 64-row decode tiles (hint 16) and on the 256-row tiles (hint 128)
        mm_dec = torch.from_numpy(synth.masked_counts(16, 32, seed + 500)).to(dev)
        ms_dec = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_masked((qa, sa), (qb, sb), d, mm_dec, 16), reps, flush)
        ms_big = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_masked((qa, sa), (qb, sb), d, mm_dec, 128), reps, flush)
        out[f"masked_decode_G16_{n}x{k}"] = {
            "rows": int(mm_dec.sum().item()), "us_64row_tiles": ms_dec * 1e3, "us_256row_tiles": ms_big * 1e3,
            "b_read_gbs_64row_tiles": b_bytes / ms_dec / 1e6, "b_read_gbs_256row_tiles": b_bytes / ms_big / 1e6,
            "hbm_gbs_counted_64row_tiles": counted_gbs(traffic, f"masked_decode_G16_{n}x{k}_64row_tiles", ms_dec * 1e3),
            "hbm_gbs_counted_256row_tiles": counted_gbs(traffic, f"masked_decode_G16_{n}x{k}_256row_tiles",
                                                        ms_big * 1e3)}
        del qa, sa, qb, sb, d
    # --- dense M=4096 shapes with power-of-two scales: fp32 scale words vs packed UE8M0 words
    shapes4k = [s for s in synth.config1_shapes() if s[0] == 4096]
    tot_flops, t_fp32, t_packed = 0.0, 0.0, 0.0
    per = {}
    for (m, n, k) in shapes4k:
        log(f"extras: dense {m}x{n}x{k}, power-of-two scales")
        seed = synth.seed_for(1, synth.config1_shapes().index((m, n, k)))
        a32 = synth.draw_activation_device(m, k, seed, dev)
        b32 = synth.draw_weight_device(n, k, seed, 0, dev)
        qa, sa = dg.per_token_cast_fp8(a32, ue8m0=True, sf=mn_major(m, k // 128, dev))
        qb, sb = dg.per_block_cast_fp8(b32, ue8m0=True)
        del a32, b32
        pa, pb = packed_mn_major(dg, sa, dev), dg.pack_ue8m0(sb)
        d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ms_f = event_time_ms(lambda: dg.fp8_gemm_nt((qa, sa), (qb, sb), d), reps, flush)
        ms_p = event_time_ms(lambda: dg.fp8_gemm_nt((qa, pa), (qb, pb), d), reps, flush)
        f = 2.0 * m * n * k
        tot_flops += f
        t_fp32 += ms_f
        t_packed += ms_p
        per[f"{m}x{n}x{k}"] = {"us_fp32_scales": ms_f * 1e3, "us_packed_ue8m0": ms_p * 1e3}
        del qa, sa, qb, sb, pa, pb, d
    out["dense_M4096_pow2_scales"] = {
        "tflops_fp32_scales": tot_flops / t_fp32 / 1e9, "tflops_packed_ue8m0": tot_flops / t_packed / 1e9,
        "pct_fp8_peak_packed_ue8m0": 100 * tot_flops / t_packed / 1e9 / FP8_PEAK_TFLOPS, "per_shape": per}
    # --- Zipf contiguous G=256, power-of-two scales
    log("extras: Zipf contiguous G=256")
    counts, m_indices = synth.config4_routing()
    n, k = synth.CONFIG4_NK
    seed = synth.seed_for(4, 0)
    m_total = m_indices.size
    valid = torch.as_tensor(np.nonzero(m_indices >= 0)[0], device=dev)
    a32 = torch.zeros((m_total, k), dtype=torch.float32, device=dev)
    a32[valid] = synth.draw_activation_device(int(valid.numel()), k, seed, dev)
    qa, sa = dg.per_token_cast_fp8(a32, ue8m0=True, sf=mn_major(m_total, k // 128, dev))
    del a32
    qb = torch.empty((256, n, k), dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty((256, (n + 127) // 128, k // 128), dtype=torch.float32, device=dev)
    for g in range(256):
        dg.per_block_cast_fp8(synth.draw_weight_device(n, k, seed, g, dev), ue8m0=True, q=qb[g], sf=sb[g])
    d = torch.empty((m_total, n), dtype=torch.bfloat16, device=dev)
    mi = torch.from_numpy(m_indices).to(dev)
    ms = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((qa, sa), (qb, sb), d, mi), max(3, reps // 2), flush)
    pa, pb = packed_mn_major(dg, sa, dev), dg.pack_ue8m0(sb)
    ms_p = event_time_ms(lambda: dg.m_grouped_fp8_gemm_nt_contiguous((qa, pa), (qb, pb), d, mi), max(3, reps // 2),
                         flush)
    useful = 2.0 * int(counts.sum()) * n * k
    ceil = ceiling_tflops(useful, min_bytes(int(counts.sum()), n, k, 256))
    out["contiguous_zipf_G256_4096x7168_ue8m0"] = {
        "ceiling_tflops": ceil, "pct_of_ceiling": 100 * useful / ms / 1e9 / ceil,
        "us": ms * 1e3, "tflops_useful": useful / ms / 1e9, "tflops_padded": 2.0 * m_total * n * k / ms / 1e9,
        "pct_fp8_peak": 100 * useful / ms / 1e9 / FP8_PEAK_TFLOPS, "b_read_gbs": 256 * n * k / ms / 1e6,
        "m_total": m_total, "us_packed_ue8m0_scales": ms_p * 1e3,
        "tflops_useful_packed_ue8m0": useful / ms_p / 1e9,
        "hbm_gbs_counted": counted_gbs(traffic, "contiguous_zipf_G256_4096x7168_ue8m0", ms * 1e3),
        "hbm_gbs_counted_packed_ue8m0": counted_gbs(traffic, "contiguous_zipf_G256_4096x7168_ue8m0_packed",
                                                    ms_p * 1e3)}
    del pa, pb
    del qa, sa, qb, sb, d
    # --- per-token cast of the bf16 activation
    x = synth.config4_cast_input().to(dev)
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev)
    s = torch.empty((x.shape[0], x.shape[1] // 128), dtype=torch.float32, device=dev)
    elems = x.numel()
    for ue in (False, True):
        ms = event_time_ms(lambda: dg.per_token_cast_fp8(x, ue8m0=ue, q=q, sf=s), reps, flush)
        nbytes = elems * (2 + 1) + elems // 128 * 4
        out[f"per_token_cast_bf16_32768x7168{'_ue8m0' if ue else ''}"] = {
            "us": ms * 1e3, "gbs": nbytes / ms / 1e6, "pct_hbm_peak": 100 * nbytes / ms / 1e6 / HBM_PEAK_GBS}
    return out


def _host_info():
    """CPU model, BLAS library and the threads it uses (threadpoolctl)."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    lib = ", ".join(sorted({"%s %s" % (i.get("internal_api", "?"), i.get("version", "")) for i in blas})) or "none"
    return model, lib, int(threads)


def cpu_baseline():
    """The oracle as it stands (decode, float64 BLAS matmul, one bf16 rounding;
    the quantizer for the cast), timed on the host cores.  The oracle's time
    does not depend on the values, so the operands are random finite E4M3 codes
    and random scales of each workload's exact shapes (drawing them is not
    timed).  Dense step: every GEMM of the workload in full, once.  MoE
    workloads: the oracle on a sample of groups, extrapolated by useful FLOPs.
    Cast: a row sample of the bf16 [32768, 7168] activation."""
    from oracle import gemm as ogemm
    from oracle import quant
    rng = np.random.default_rng(7)

    def codes(shape):
        return (rng.integers(0, 0x7F, size=shape, dtype=np.uint8) | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7))

    def scales(shape):
        return np.exp2(rng.uniform(-12, -4, size=shape)).astype(np.float32)

    per = {}
    # dense step, every GEMM in full
    t_step, flops_step = 0.0, 0.0
    for (m, n, k) in synth.config1_shapes():
        qa, sa, qb, sb = codes((m, k)), scales((m, k // 128)), codes((n, k)), scales(((n + 127) // 128, k // 128))
        t0 = time.perf_counter()
        ogemm.gemm_nt(qa, sa, qb, sb)
        t_step += time.perf_counter() - t0
        flops_step += 2.0 * m * n * k
        del qa, sa, qb, sb
    per["dense_step"] = {"s": round(t_step, 3), "tflops": round(flops_step / t_step / 1e12, 4), "sample": "all 15 GEMMs"}
    # config 0
    qa, sa, qb, sb = codes((128, 512)), scales((128, 4)), codes((256, 512)), scales((2, 4))
    t0 = time.perf_counter()
    ogemm.gemm_nt(qa, sa, qb, sb)
    dt = time.perf_counter() - t0
    per["dense_128x256x512"] = {"s": round(dt, 5), "tflops": round(2.0 * 128 * 256 * 512 / dt / 1e12, 5)}

    def grouped(name, counts, n, k, sample_groups, masked):
        """oracle time on the rows of sample_groups, extrapolated by useful FLOPs"""
        rows = [int(counts[g]) for g in sample_groups]
        r = sum(rows)
        qa, sa = codes((r, k)), scales((r, k // 128))
        qb, sb = codes((len(rows), n, k)), scales((len(rows), (n + 127) // 128, k // 128))
        t0 = time.perf_counter()
        if masked:
            mm = max(rows)
            a3 = np.zeros((len(rows), mm, k), np.uint8)
            s3 = np.ones((len(rows), mm, k // 128), np.float32)
            ogemm.m_grouped_masked(a3, s3, qb, sb, np.array(rows, np.int32))
        else:
            mi = np.concatenate([np.full(c, i, np.int32) for i, c in enumerate(rows)])
            ogemm.m_grouped_contiguous(qa, sa, qb, sb, mi)
        dt = time.perf_counter() - t0
        useful_sample = 2.0 * r * n * k
        useful = 2.0 * int(np.sum(counts)) * n * k
        per[name] = {"s_extrapolated": round(dt * useful / useful_sample, 3),
                     "tflops": round(useful_sample / dt / 1e12, 4),
                     "sample": "%d of %d groups (%d rows)" % (len(rows), len(counts), r)}

    for idx, (n, k) in enumerate(synth.GROUPED_NK):
        counts, _ = synth.config2_routing(idx)
        grouped(f"contiguous_G8_{n}x{k}", counts, n, k, [0, 1], False)
        mm = synth.config3_masked_m(idx)
        grouped(f"masked_G16_{n}x{k}", mm, n, k, [int(np.argmax(mm)), 0], True)
    counts, _ = synth.config4_routing()
    n, k = synth.CONFIG4_NK
    order = np.argsort(counts)
    grouped("contiguous_zipf_G256_4096x7168", counts, n, k, [int(order[-1]), int(order[len(order) // 2]),
                                                              int(order[0])], False)
    # cast: 1024 rows of the bf16 activation (widened exactly to fp32)
    x = (rng.standard_normal((1024, 7168)) * np.exp2(rng.uniform(-4, 4, (1024, 1)))).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    t0 = time.perf_counter()
    quant.per_token_cast(x)
    dt = time.perf_counter() - t0
    per["per_token_cast_bf16"] = {"gbs": round(x.size * (2 + 1 + 4 / 128) / dt / 1e9, 4),
                                  "sample": "1024 of 32768 rows"}
    model, lib, threads = _host_info()
    return {"value": round(flops_step / t_step / 1e12, 4), "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": "the whole dense workload (all 15 GEMMs at full size, once) through the oracle: "
                      "%.1f s; random E4M3 codes and scales of the exact shapes" % t_step,
            "cpu_model": model, "blas": lib, "host_cores": len(os.sched_getaffinity(0)), "per_config": per}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dense_gemm.txt")
# The GEMM kernels' source: the kernel file and the two headers it includes.
GEMM_SOURCES = [os.path.join(ROOT, "moe_fp8_gemm_amd", "csrc", f)
                for f in ("gemm_fp8.hip", "dgfp8_device.h", "dgfp8_internal.h")]


def gemm_source_sha256():
    """sha256 of the GEMM kernel sources, concatenated in the order above."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_profile(cfg, shapes):
    """Counter figures of the dominant instance from the committed PMC summary:
    HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated against a 1 GiB
    copy) and the shader clock it ran at (GRBM_GUI_ACTIVE).  None when there is
    none for this instance and shape set or the kernel source has changed since
    the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    sha = gemm_source_sha256()
    want_shapes = ",".join("%dx%dx%d" % s for s in shapes)
    if (kv.get("kernel_source_sha256") != sha or kv.get("tile") != "%dx%dx%d" % cfg
            or kv.get("shapes") != want_shapes):
        return None
    return kv


TRAFFIC_ROWS_FILE = os.path.join(ROOT, "profiles", "traffic_hbm_bound.txt")


def counted_traffic():
    """{row: calibrated HBM bytes per call} from the committed counter summary of
    the HBM-bound rows (FETCH_SIZE / calibration + WRITE_SIZE / calibration, in
    bytes); empty when the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_ROWS_FILE):
        return {}
    kv = {}
    for line in open(TRAFFIC_ROWS_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    if kv.pop("kernel_source_sha256", None) != gemm_source_sha256():
        return {}
    fc, wc = float(kv.pop("fetch_calibration")), float(kv.pop("write_calibration"))
    out = {}
    for row, val in kv.items():
        fetch, write = (float(x) for x in val.split())
        out[row] = (fetch / fc + write / wc) * 1024
    return out


def counted_gbs(traffic, row, us):
    """Counted HBM GB/s of one call of `row` that took `us` microseconds (None
    without a valid counter figure)."""
    return round(traffic[row] / (us * 1e-6) / 1e9, 1) if row in traffic and us > 0 else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="profiling aid: after the timed steps, copy a 1 GiB buffer 3 times (a kernel of known "
                         "traffic, to calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--only", default=None,
                    help="profiling aid: time only this M,N,K of the workload (e.g. 4096,4096,7168)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU; multi-GPU (expert-parallel) runs are not "
              "implemented -- use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import moe_fp8_gemm_amd as dg

    dev = torch.device("cuda:0")
    shapes = synth.config1_shapes()
    if args.only:
        want = tuple(int(x) for x in args.only.split(","))
        if want not in shapes:
            sys.exit(f"--only {args.only} is not one of the workload's shapes")
        shapes = [want]
    log("preparing inputs")
    probs = []
    for (m, n, k) in shapes:
        idx = synth.config1_shapes().index((m, n, k))
        probs.append(make_dense(dg, m, n, k, synth.seed_for(1, idx), dev))
    torch.cuda.synchronize()
    flops = [2.0 * m * n * k for (m, n, k) in shapes]

    # Which (tile, split) instance runs each launch: the plan is a pure function
    # of the shape.  The dominant instance is the one that takes most of the step.
    cfgs = [dg.tile_config(m, n, k) for (m, n, k) in shapes]

    def step(marks=None):
        """One pass over the workload.  marks: {launch index: (start event or
        None, end event or None)} recorded around those launches only."""
        for i, (a, b, d) in enumerate(probs):
            if marks and i in marks and marks[i][0] is not None:
                marks[i][0].record()
            dg.fp8_gemm_nt(a, b, d)
            if marks and i in marks and marks[i][1] is not None:
                marks[i][1].record()

    def new_event():
        return torch.cuda.Event(enable_timing=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- per-launch times, from separate (untimed) steps with an event pair
    # around every launch.  Events cost GPU time between launches, so the timed
    # steps below carry only the few the roofline needs.
    probe_steps = max(3, min(args.steps, 10))
    probe = [{i: (new_event(), new_event()) for i in range(len(shapes))} for _ in range(probe_steps)]
    for s in range(probe_steps):
        step(probe[s])
    torch.cuda.synchronize()
    per_launch = np.array([[probe[s][i][0].elapsed_time(probe[s][i][1]) for i in range(len(shapes))]
                           for s in range(probe_steps)])      # ms
    mean_ms = per_launch.mean(axis=0)
    by_cfg = {}
    for i, c in enumerate(cfgs):
        by_cfg.setdefault(c, []).append(i)
    dom_cfg = max(by_cfg, key=lambda c: sum(mean_ms[i] for i in by_cfg[c]))
    big = by_cfg[dom_cfg]
    # runs of consecutive launches of the dominant instance: one event pair per run
    runs, cur = [], [big[0]]
    for i in big[1:]:
        if i == cur[-1] + 1:
            cur.append(i)
        else:
            runs.append(cur)
            cur = [i]
    runs.append(cur)

    # ---- timed steps: wall clock over the whole job; HIP events on the launch
    # stream bracket each run of dominant-instance launches
    log(f"timing {args.steps} steps")
    marks = []
    for _ in range(args.steps):
        mk = {}
        for r in runs:
            e0, e1 = new_event(), new_event()
            mk[r[0]] = (e0, mk.get(r[0], (None, None))[1])
            mk[r[-1]] = (mk.get(r[-1], (None, None))[0], e1)
        marks.append(mk)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(marks[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12
    # The dominant kernel's achieved rate = algorithmic FLOPs per launch / average
    # launch duration (event time of its runs over the timed steps / launches).
    dom_total_ms = sum(marks[s][r[0]][0].elapsed_time(marks[s][r[-1]][1]) for s in range(args.steps) for r in runs)
    dom_time = dom_total_ms / (args.steps * len(big))
    dom_flops = float(np.mean([flops[i] for i in big]))
    achieved = dom_flops / (dom_time * 1e-3) / 1e12
    # Operand bytes the dominant instance stages from L2 into LDS per launch:
    # every tile copies its A rows and B rows of each 128-wide K block once.
    bm, bn = dom_cfg[0], dom_cfg[1]
    staged = float(np.mean([math.ceil(shapes[i][0] / bm) * math.ceil(shapes[i][1] / bn) * (shapes[i][2] // 128)
                            * (bm + bn) * 128 for i in big]))
    if args.calib_copy:
        src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    per_shape = []
    for i, (m, n, k) in enumerate(shapes):
        per_shape.append({"m": m, "n": n, "k": k, "us_in_step": float(mean_ms[i] * 1e3),
                          "tflops": flops[i] / (mean_ms[i] * 1e-3) / 1e12})
    log("cold-cache per-shape times")
    flush = Flusher(dev)
    traffic = counted_traffic()
    for i, (a, b, d) in enumerate(probs):
        ms = event_time_ms(lambda: dg.fp8_gemm_nt(a, b, d), 10, flush)
        per_shape[i]["us_cold"] = ms * 1e3
        per_shape[i]["tflops_cold"] = flops[i] / (ms * 1e-3) / 1e12
        per_shape[i]["pct_fp8_peak_cold"] = 100 * per_shape[i]["tflops_cold"] / FP8_PEAK_TFLOPS
        ceil = ceiling_tflops(flops[i], min_bytes(*shapes[i]))
        per_shape[i]["ceiling_tflops"] = ceil
        per_shape[i]["ceiling_us"] = flops[i] / (ceil * 1e12) * 1e6
        per_shape[i]["pct_of_ceiling_cold"] = 100 * per_shape[i]["tflops_cold"] / ceil
        if shapes[i][0] <= 128:
            per_shape[i]["hbm_gbs_counted_cold"] = counted_gbs(traffic, "%dx%dx%d" % shapes[i], ms * 1e3)
            # Back-to-back launches over enough distinct operand copies (> 512 MB
            # in all) that every launch still reads its operands from HBM: the
            # per-launch event overhead is paid once per batch, not per launch.
            # The flush object above stays alive; this one adds 1 GiB briefly.
            us = pipelined_cold_us(dg, a, b, d)
            per_shape[i]["us_cold_pipelined"] = us
            per_shape[i]["pct_of_ceiling_cold_pipelined"] = 100 * flops[i] / (us * 1e-6) / 1e12 / ceil
    del flush
    floor_us = event_floor_us(dev)
    prof = measured_profile(dom_cfg, [shapes[i] for i in big])
    # The 5.0 PFLOP/s peak assumes 2.4 GHz (256 CUs x 8192 FP8 FLOP per clock);
    # the committed counter pass also gives the clock the kernel actually ran at.
    sclk = float(prof["sclk_ghz"]) if prof and "sclk_ghz" in prof else None
    peak_at_sclk = 256 * 8192 * sclk / 1e3 if sclk else None
    result = {
        "metric": "FP8 block-scaled GEMM TFLOPS (1 GPU) and % of MI355X FP8 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded device-side N(0,1) draws, log-uniform row factors; quantized by the library casts)",
        "config": {"workload": "dense fp8_gemm_nt, LLM-layer shapes: M in {64,128,4096} x (N,K) in "
                               "{(2112,7168),(24576,1536),(7168,16384),(4096,7168),(7168,2048)}; "
                               "A 1x128 and B 128x128 fp32 block scales, bf16 out",
                   "gemms_per_step": len(shapes), "pct_fp8_peak": round(100 * value / FP8_PEAK_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": int(float(prof["hbm_bytes_per_launch"])) if prof else None,
                     "kernel": "dense %dx%d-tile GEMM%s" % (dom_cfg[0], dom_cfg[1],
                                                            "" if dom_cfg[2] == 1 else ", split-K %d" % dom_cfg[2]),
                     "shapes": ["%dx%dx%d" % shapes[i] for i in big],
                     "avg_launch_us": round(dom_time * 1e3, 2), "flops_per_launch": dom_flops,
                     "staged_bytes_per_launch": int(staged),
                     "staged_gbs_per_cu": round(staged / (dom_time * 1e-3) / 1e9 / 256, 1),
                     "sclk_ghz_profiled": sclk,
                     "peak_at_profiled_sclk": round(peak_at_sclk, 1) if sclk else None,
                     "frac_at_profiled_sclk": round(achieved / peak_at_sclk, 4) if sclk else None},
        "per_shape": per_shape,
        "event_floor_us": round(floor_us, 2),
    }
    if not args.no_extras:
        log("extras: MoE workloads and cast")
        del probs
        torch.cuda.empty_cache()
        result["extras"] = bench_extras(dg, dev, reps=10)
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
