"""Benchmark of the HYPIC linear-layer hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  main workload  GDN, H=32, d_k=d_v=128, bf16 k/v, fp32 records: one 32768-token
                 request split into 16 segments of 2048 tokens; build all 512
                 (segment, head) records, then compose the 16-segment chain to
                 the request's final state.
Secondary lines (same JSON object, key "secondary"):
  forward        the same workload's chunked prefill forward (in-segment outputs
                 o_t = S_t^T q_t, bf16 q and o) alone and with the records as
                 side-outputs: the records' cost as a fraction of the forward
  compose_pool   4096-slot GDN pool (H=32, d=128, fp32 records), 64 requests each
                 composing 32 seeded slot ids -> compositions/s
  scalar/diag    RetNet-style scalar and GLA-style diagonal builds, H=16, d=128,
                 bf16, 8 x 2048 tokens, plus their 8-segment chains
  rag mix        128 requests of 24-96 cached/cold GDN segments (128-1024 tokens),
                 cold builds + conv warm-up (4096 channels, kernel 4) + all chains
  conv exact     conv-coupled exact reuse: 32 requests of 24-96 cached segments,
                 warmed head keys/values applied inside the compose
  kda            KDA family build (chunked, on the fp32 matrix cores) and its
                 8-segment chain, H=16, d=128, bf16, 8 x 2048 tokens
  peaks          measured peaks of this machine: a streaming read and a loop of bf16
                 matrix-core products (libhypic_peaks.so)

Inputs are resident in HBM before the timed region starts.  Kernel durations
come from HIP events recorded on the stream the kernels are launched on, one
event pair per launch (mean, p10, p50, p90 reported).  The cpu_baseline leg
times the fp64 oracle on a bounded sample on the host.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only main|forward|sd|compose|rag|convexact|kda|peaks] [--no-cpu]
       python bench.py --summarize-traffic FETCH_CSV WRITE_CSV OUT_DIR  (rocprofv3 counter CSVs -> summaries)
       python bench.py --summarize-mfma CSV OUT_MD
       python bench.py --summarize-trace TRACE_CSV STATS_CSV BENCH_JSON OUT_MD
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import hybrid_prefill_amd as hp  # noqa: E402
import synth  # noqa: E402

METRIC = "segment-build tokens/s + segment compositions/s at GDN H=32,d=128; % MFMA/HBM peak"
PEAK_HBM = 8.0e12            # B/s, MI355X published
PEAK_BF16 = 2.5e15           # FLOP/s dense bf16 MFMA
PEAK_FP32 = 157.3e12         # FLOP/s fp32 (matrix and vector, published)
CHUNK = 64
CSRC = os.path.join(ROOT, "hybrid_prefill_amd", "csrc")
# HBM bytes per launch of each timed kernel come from committed rocprofv3 counter
# summaries (FETCH_SIZE and WRITE_SIZE, scaled by what the counters read for a device
# copy of known size in the same process).  Each summary records a hash of the
# kernel's sources; when they have changed since, the bytes are unknown (null) until
# the counters are taken again.  key -> (kernel name fragment, grid in threads as the
# counter CSV reports it (None: any), bench phase (see PHASES), sources, workload)
_GDN_SRC = ("build_mfma.hip", "gdn_mfma_common.h", "hypic_internal.h")
_FWD_SRC = ("build_fwd_mfma.hip", "gdn_mfma_common.h", "hypic_internal.h")
_CMP_SRC = ("compose_mfma.hip", "hypic_internal.h")
_SD_SRC = ("build_sd_mfma.hip", "hypic_internal.h")
TRAFFIC_KERNELS = {
    "gdn_build_h32_d128_16x2048": ("gdn_build_mfma_kernel(", None, "main", _GDN_SRC,
                                   "GDN build, H=32, d=128, bf16, 16 x 2048 tokens"),
    "gdn_compose_h32_d128_chain16": ("compose_sliced_mfma_kernel", 65536, "main", _CMP_SRC,
                                     "GDN compose of the 16-segment chain, H=32, d=128, fp32 records"),
    "gdn_forward_h32_d128_16x2048": ("gdn_chunk_mfma_kernel<false, true>", 262144, "forward", _FWD_SRC,
                                     "GDN prefill forward, outputs only, H=32, d=128, bf16, 16 x 2048 tokens"),
    "gdn_forward_records_h32_d128_16x2048": ("gdn_chunk_mfma_kernel<true, true>", 393216, "forward", _FWD_SRC,
                                             "GDN prefill forward with record side-outputs, H=32, d=128, bf16, "
                                             "16 x 2048 tokens"),
    "gdn_compose_pool4096_h32_d128_64x32": ("compose_dense_mfma_kernel<false, false>", 524288, "compose", _CMP_SRC,
                                            "GDN compose, 4096-slot pool, 64 requests x 32 slots, H=32, d=128"),
    "scalar_build_h16_d128_8x2048": ("sd_build_mfma_kernel<0, 2>", 131072, "sd", _SD_SRC,
                                     "scalar-decay build, H=16, d=128, bf16, 8 x 2048 tokens"),
    "diagonal_build_h16_d128_8x2048": ("sd_build_mfma_kernel<1, 2>", 196608, "sd", _SD_SRC,
                                       "diagonal-gate build, H=16, d=128, bf16, 8 x 2048 tokens"),
    "conv_warmup_rag_8305x4096_k4": ("conv_warmup_vec_kernel", None, "rag", ("conv_warmup.hip", "hypic_internal.h"),
                                     "conv warm-up of the RAG mix, 8305 boundaries x 4096 channels, kernel 4, bf16"),
    "gdn_build_rag_cold_2584seg": ("gdn_build_mfma_kernel(", None, "rag", _GDN_SRC,
                                   "GDN build of the RAG mix's 2584 cold segments (128-1024 tokens), H=32, d=128"),
    "gdn_compose_rag_128req": ("compose_dense_mfma_kernel<false, false>", 1048576, "rag", _CMP_SRC,
                               "GDN compose of the RAG mix's 128 chains (24-96 slots), H=32, d=128"),
}

# Bench phases.  The GDN build runs the same grid (a multiple of the CU count) for
# every workload above a few hundred (segment, head) units, so a profile cannot tell
# the legs apart by kernel and grid; each leg, and the untimed set-up inside a leg,
# therefore starts with a marker launch: the streaming-copy microbenchmark over 16
# bytes with as many 512-thread workgroups as the phase's position in PHASES (plus
# one).  The profile summaries attribute every dispatch to the last marker before it.
PHASES = ("main", "forward", "compose_setup", "compose", "sd", "rag_setup", "rag", "convexact_setup", "convexact",
          "kda", "peaks")
_PEAKS = None
_MARK_BUF = None


def peaks_lib():
    """libhypic_peaks.so: the measured-peak microbenchmarks (outside the library's ABI)."""
    global _PEAKS
    if _PEAKS is None:
        from hybrid_prefill_amd import _build
        L = ctypes.CDLL(_build.PEAKS_LIB)
        L.hypic_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
        L.hypic_peak_mfma.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.hypic_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_void_p]
        _PEAKS = L
    return _PEAKS


def mark(phase):
    """The marker launch of a bench phase, on the current stream."""
    global _MARK_BUF
    if _MARK_BUF is None:
        _MARK_BUF = torch.zeros(8, dtype=torch.float32, device="cuda")
    rc = peaks_lib().hypic_peak_copy(_MARK_BUF.data_ptr(), _MARK_BUF.data_ptr() + 16, 16, PHASES.index(phase) + 1,
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == 0, "marker launch failed"


def dispatch_phases(rows):
    """rows: (dispatch id, kernel name, grid in threads, ...) in any order -> {dispatch id:
    phase or None}, markers themselves left out."""
    phase, out = None, {}
    for r in sorted(rows, key=lambda t: t[0]):
        did, name, grid = r[0], r[1], r[2]
        if "peak_copy_kernel" in name and grid % 512 == 0 and 1 <= grid // 512 <= len(PHASES):
            phase = PHASES[grid // 512 - 1]
            continue
        out[did] = phase
    return out


def source_sha(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_profile(key) -> str:
    return os.path.join(ROOT, "profiles", f"{key}_traffic.md")


def committed_traffic(key="gdn_build_h32_d128_16x2048"):
    """HBM bytes per launch from the committed counter summary, or None when it is
    missing or the kernel's sources changed since it was taken."""
    if key not in TRAFFIC_KERNELS:
        return None
    try:
        text = open(traffic_profile(key)).read()
    except OSError:
        return None
    m_sha = re.search(r"kernel source sha256\[:16\]: `([0-9a-f]{16})`", text)
    m_tot = re.search(r"HBM bytes per launch: ([0-9.]+) MB", text)
    if not (m_sha and m_tot) or m_sha.group(1) != source_sha(TRAFFIC_KERNELS[key][3]):
        return None
    return float(m_tot.group(1)) * 1e6


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic counts

def gdn_build_flops_per_token_head(dk, dv, c=CHUNK):
    """Gram (strict lower triangle) + triangular solves on the right-hand sides of
    the P and S columns + the inter-chunk carry (Z = K X and the rank-c update, for
    P and S)."""
    return (c - 1) * dk + (c - 1) * (dk + dv) + 4 * dk * (dk + dv)


def gdn_build_bytes(N, H, dk, dv, nseg, kv_bytes=2):
    tokens = N * H * (kv_bytes * (dk + dv) + 4 + 4)          # k, v, beta, log alpha
    records = nseg * H * 4 * (dk * dk + dk * dv + 1)          # P, S, ell
    return tokens + records


def sd_build_bytes(family, N, H, dk, dv, nseg, kv_bytes=2):
    gates = 4 * dk if family == hp.DIAGONAL else 0            # per-token gates (diagonal); scalar: per head
    tokens = N * H * (kv_bytes * (dk + dv) + gates)
    ell = dk if family == hp.DIAGONAL else 1
    return tokens + nseg * H * 4 * (dk * dv + ell)


def compose_bytes(chain_lengths, H, dk, dv, family=hp.GDN):
    """Per (request, head): every record's S and ell, the P of every record but
    the first (the first acts on a zero state), and the output S."""
    ell = dk if family == hp.DIAGONAL else 1
    per_P = dk * dk if family == hp.GDN else 0
    total = 0
    for m in chain_lengths:
        if m == 0:
            total += H * 4 * dk * dv
            continue
        total += H * 4 * (m * (dk * dv + ell) + (m - 1) * per_P + dk * dv)
    return total


# ----------------------------------------------------------------------------- timing helpers

class KernelTimer:
    """Accumulates HIP-event durations of launches on the current stream."""

    def __init__(self):
        self.pairs = {}

    def time(self, name, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return out

    def mean_ms(self, name):
        torch.cuda.synchronize()
        ts = [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]
        return float(np.mean(ts)) if ts else float("nan")

    def reset(self):
        self.pairs = {}


def launch_stats(launches, n):
    """Per-launch durations of each launch in `launches` (name -> callable, idempotent):
    one HIP-event pair around every launch on the current stream, after a short device
    spin that lets the host queue the launches ahead, so that no host time between an
    event and its launch counts as kernel time.  Returns {name: stats}."""
    out = {}
    for name, fn in launches:
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(5e6))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for s_, e_ in ev:
            s_.record()
            fn()
            e_.record()
        torch.cuda.synchronize()
        out[name] = stats_ms([s_.elapsed_time(e_) for s_, e_ in ev])
    return out


def stats_ms(ts):
    a = np.asarray(ts, dtype=np.float64)
    return {"mean": float(a.mean()), "p10": float(np.percentile(a, 10)), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def kernel_pass(launches, n):
    """Mean duration of each launch (see launch_stats)."""
    st = launch_stats(launches, n)
    return tuple(st[name]["mean"] for name, _ in launches)


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic}


# ----------------------------------------------------------------------------- workloads

def gdn_workload(H=32, dk=128, dv=128, nseg=16, seg_len=2048, seed=301):
    st = synth.gdn_stream([seg_len] * nseg, H, dk, dv, torch.bfloat16, seed, 0.1, "cuda")
    pool = hp.Pool.allocate(hp.GDN, nseg, H, dk, dv, device="cuda")
    return dict(st=st, pool=pool, offs=torch.as_tensor(st.seg_offsets).cuda(),
                slots=torch.arange(nseg, dtype=torch.int32, device="cuda"),
                chain_offs=torch.tensor([0, nseg], dtype=torch.int64, device="cuda"),
                out_S=torch.empty((1, H, dk, dv), device="cuda"),
                err=torch.zeros(1, dtype=torch.int32, device="cuda"),
                H=H, dk=dk, dv=dv, nseg=nseg, seg_len=seg_len, N=nseg * seg_len)


def gdn_step(w):
    """One step of the hot path: every record of the batch built, then the chain composed."""
    st, pool = w["st"], w["pool"]
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, w["offs"], pool, w["slots"], beta=st.beta,
                     err_flag=w["err"])
    hp.compose_chain(pool, w["chain_offs"], w["slots"], out_S=w["out_S"], err_flag=w["err"])


def capture_step(w):
    """The step's two launches captured once into a HIP graph (torch.cuda.CUDAGraph over
    the library's launches on the capturing stream; the step makes no allocation, copy,
    memset or host synchronisation).  Replays run the same kernels on the same buffers."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gdn_step(w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn_step(w)
    torch.cuda.synchronize()
    return g


def timed_steps(run, steps):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def bench_main(args):
    mark("main")
    w = gdn_workload()
    for _ in range(args.warmup):
        gdn_step(w)
    ms_eager = timed_steps(lambda: gdn_step(w), args.steps)
    assert int(w["err"].item()) == 0
    # the headline step: the same two launches replayed from a HIP graph (no launch gap
    # between the build and the compose beyond the graph's own)
    g = capture_step(w)
    for _ in range(args.warmup):
        g.replay()
    ms_step = timed_steps(g.replay, args.steps)
    assert int(w["err"].item()) == 0
    w["ms_eager"] = ms_eager
    del g
    # per-kernel durations: the same steps again, one event pair per launch with the
    # launch queue filled ahead (a short device spin first)
    st_, pool_ = w["st"], w["pool"]
    ks = launch_stats((
        ("build", lambda: hp.build_segment(hp.GDN, st_.k, st_.v, st_.log_alpha, w["offs"], pool_, w["slots"],
                                           beta=st_.beta, err_flag=w["err"])),
        ("compose", lambda: hp.compose_chain(pool_, w["chain_offs"], w["slots"], out_S=w["out_S"],
                                             err_flag=w["err"]))), max(args.steps, 10))
    b_ms, c_ms = ks["build"]["mean"], ks["compose"]["mean"]
    N, H, dk, dv, nseg = w["N"], w["H"], w["dk"], w["dv"], w["nseg"]
    flops = gdn_build_flops_per_token_head(dk, dv) * N * H
    bbytes = gdn_build_bytes(N, H, dk, dv, nseg)
    cbytes = compose_bytes([nseg], H, dk, dv)
    log(f"main: {ms_step:.3f} ms/step wall (graph replay; eager launches {ms_eager:.3f}); build {b_ms:.3f} ms (p10 {ks['build']['p10']:.3f}, "
        f"p90 {ks['build']['p90']:.3f}), compose {c_ms:.3f} ms; build {flops / (b_ms * 1e-3) / 1e12:.1f} TFLOP/s, "
        f"{bbytes / (b_ms * 1e-3) / 1e9:.0f} GB/s")
    kern = {
        "gdn_build": {"ms": b_ms, "ms_stats": ks["build"], "algorithmic_flop": flops, "algorithmic_bytes": bbytes,
                      "tflops": flops / (b_ms * 1e-3) / 1e12, "gbps": bbytes / (b_ms * 1e-3) / 1e9,
                      "tokens_per_s": N / (b_ms * 1e-3)},
        "gdn_compose_chain16": {"ms": c_ms, "ms_stats": ks["compose"], "algorithmic_bytes": cbytes,
                                "gbps": cbytes / (c_ms * 1e-3) / 1e9, "compositions_per_s": nseg / (c_ms * 1e-3),
                                "traffic": committed_traffic("gdn_compose_h32_d128_chain16")},
    }
    return ms_step, N, kern, flops, b_ms, w


def forward_bytes(N, H, dk, dv, nseg, o_bytes=2, records=False, kv_bytes=2):
    """k, q, v (kv_bytes each), beta and log alpha (fp32), the outputs; plus the records."""
    b = N * H * (kv_bytes * (2 * dk + dv) + 8 + o_bytes * dv)
    if records:
        b += nseg * H * 4 * (dk * dk + dk * dv + 1)
    return b


def bench_forward(args, w, build_ms):
    """The main workload's chunked prefill forward (in-segment outputs, bf16 q and o)
    alone and with the records as side-outputs; beside them the record build alone
    (the main leg's kernel).  besthub article, paragraph 7: the records' one-time
    construction costs a small fraction of a forward pass."""
    mark("forward")
    st, pool = w["st"], w["pool"]
    N, H, dk, dv, nseg = w["N"], w["H"], w["dk"], w["dv"], w["nseg"]
    q = synth.keys(N, H, dk, torch.bfloat16, 3017, "cuda")
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    fwd = lambda: hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, w["offs"], beta=st.beta, out=o)
    fwd_rec = lambda: hp.prefill_segment(hp.GDN, st.k, st.v, q, st.log_alpha, w["offs"], beta=st.beta, out=o,
                                         pool=pool, dst_slots=w["slots"])
    for _ in range(max(1, args.warmup)):
        fwd()
        fwd_rec()
    ks = launch_stats((("forward", fwd), ("forward_records", fwd_rec)), max(args.steps, 10))
    f_ms, fr_ms = ks["forward"]["mean"], ks["forward_records"]["mean"]
    fb = forward_bytes(N, H, dk, dv, nseg)
    frb = forward_bytes(N, H, dk, dv, nseg, records=True)
    log(f"forward: {f_ms:.3f} ms ({fb / (f_ms * 1e-3) / 1e9:.0f} GB/s), with records {fr_ms:.3f} ms "
        f"(+{100 * (fr_ms / f_ms - 1):.1f} %), records alone {build_ms:.3f} ms")
    del q, o
    return {"workload": "gdn_prefill_forward_h32_d128_bf16_16x2048", "metric": "tokens/s",
            "value": N / (f_ms * 1e-3), "unit": "tokens/s", "ms": f_ms, "ms_stats": ks["forward"],
            "with_records": {"ms": fr_ms, "ms_stats": ks["forward_records"], "tokens_per_s": N / (fr_ms * 1e-3)},
            "record_side_output_cost_frac": fr_ms / f_ms - 1.0,
            "record_build_alone_frac": build_ms / f_ms,
            "roofline": roofline("hbm", fb / (f_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s",
                                  committed_traffic("gdn_forward_h32_d128_16x2048")),
            "roofline_with_records": roofline("hbm", frb / (fr_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s",
                                               committed_traffic("gdn_forward_records_h32_d128_16x2048"))}


def bench_compose_pool(args, slots=4096, H=32, d=128, R=64, m=32, seg_len=64, seed=401):
    """Pool of GDN records (filled untimed by the build), R requests x m slot ids."""
    mark("compose_setup")
    st = synth.gdn_stream([seg_len] * slots, H, d, d, torch.bfloat16, seed, 0.01, "cuda")
    pool = hp.Pool.allocate(hp.GDN, slots, H, d, d, device="cuda")
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, torch.as_tensor(st.seg_offsets).cuda(), pool,
                     torch.arange(slots, dtype=torch.int32, device="cuda"), beta=st.beta)
    del st
    torch.cuda.synchronize()
    mark("compose")
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = torch.as_tensor(rng.integers(0, slots, size=R * m).astype(np.int32)).cuda()
    offs = torch.arange(0, R * m + 1, m, dtype=torch.int64, device="cuda")
    out = torch.empty((R, H, d, d), device="cuda")
    timer = KernelTimer()
    for _ in range(args.warmup):
        hp.compose_chain(pool, offs, ids, out_S=out)
    torch.cuda.synchronize()
    for _ in range(max(3, args.steps // 2)):
        timer.time("compose", lambda: hp.compose_chain(pool, offs, ids, out_S=out))
    ms = timer.mean_ms("compose")
    nbytes = compose_bytes([m] * R, H, d, d)
    comps = R * m
    log(f"compose_pool: {ms:.3f} ms, {comps / (ms * 1e-3):.3e} compositions/s, {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    del pool
    torch.cuda.empty_cache()
    return {"workload": f"gdn_compose_pool{slots}_h{H}_d{d}_{R}x{m}", "metric": "compositions/s",
            "value": comps / (ms * 1e-3), "unit": "compositions/s", "ms": ms,
            "roofline": roofline("hbm", nbytes / (ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s",
                                  committed_traffic(f"gdn_compose_pool{slots}_h{H}_d{d}_{R}x{m}"))}


def bench_sd(args, H=16, d=128, nseg=8, seg_len=2048, seed=201, copies=3):
    """Scalar and diagonal builds + their 8-segment chains.  The inputs are
    rotated over `copies` seeded copies so that the timed working set exceeds
    the 256 MB Infinity Cache (one copy of k, v and the gates would fit)."""
    mark("sd")
    out = []
    N = nseg * seg_len
    ks = [synth.keys(N, H, d, torch.bfloat16, seed * 10 + 1 + 100 * c, "cuda") for c in range(copies)]
    vs = [synth.values(N, H, d, torch.bfloat16, seed * 10 + 2 + 100 * c, "cuda") for c in range(copies)]
    offs = torch.as_tensor(synth.even_offsets(nseg, seg_len)).cuda()
    slots = torch.arange(nseg, dtype=torch.int32, device="cuda")
    chain = torch.tensor([0, nseg], dtype=torch.int64, device="cuda")
    for fam, name in ((hp.SCALAR, "scalar"), (hp.DIAGONAL, "diagonal")):
        las = ([synth.scalar_log_gamma(H, seed * 10 + 4 + 100 * c, device="cuda") for c in range(copies)]
               if fam == hp.SCALAR else
               [synth.diagonal_log_gates(N, H, d, seed * 10 + 4 + 100 * c, device="cuda") for c in range(copies)])
        pool = hp.Pool.allocate(fam, nseg, H, d, d, device="cuda")
        for i in range(args.warmup):
            c = i % copies
            hp.build_segment(fam, ks[c], vs[c], las[c], offs, pool, slots)
        torch.cuda.synchronize()
        it = [0]

        def build_rot():
            c = it[0] % copies
            it[0] += 1
            hp.build_segment(fam, ks[c], vs[c], las[c], offs, pool, slots)
        b_ms, c_ms = kernel_pass((("build", build_rot), ("compose", lambda: hp.compose_chain(pool, chain, slots))),
                                 max(3, args.steps))
        nb = sd_build_bytes(fam, N, H, d, d, nseg)
        log(f"{name}: build {b_ms:.3f} ms ({nb / (b_ms * 1e-3) / 1e9:.0f} GB/s), compose {c_ms:.3f} ms")
        out.append({"workload": f"{name}_build_h{H}_d{d}_{nseg}x{seg_len}", "metric": "tokens/s",
                    "value": N / (b_ms * 1e-3), "unit": "tokens/s", "ms": b_ms, "compose_ms": c_ms,
                    "roofline": roofline("hbm", nb / (b_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s",
                                          committed_traffic(f"{name}_build_h{H}_d{d}_{nseg}x{seg_len}"))})
        del las, pool
    return out


def conv_bytes(B, C, K, x_bytes=2):
    return B * (2 * (K - 1) * C * x_bytes + (K - 1) * C * 4) + C * K * 4


def rag_chains(plan, R, pool_slots):
    """Slot chains of the RAG mix: cached positions name their pool slot, cold ones
    a fresh slot after the pool (cold_len: {slot: tokens})."""
    chains, cold_len, j = [], {}, 0
    for r in range(R):
        ch = []
        for pos in range(plan.chain_lengths[r]):
            if plan.is_cached[r][pos]:
                ch.append(int(plan.cached_slot[r][pos]))
            else:
                cold_len[pool_slots + j] = int(plan.cold_lengths[j])
                ch.append(pool_slots + j)
                j += 1
        chains.append(np.asarray(ch, dtype=np.int32))
    return chains, cold_len


def bench_rag(args, R=128, pool_slots=4096, H=32, d=128, C=4096, K=4, seed=501):
    """RAG-shaped step: 128 requests of 24-96 segments (128-1024 tokens), 70 %
    cache hits from a 4096-slot pool built untimed, 30 % cold segments built in
    the step, conv warm-up at every boundary, all chains composed."""
    mark("rag_setup")
    from hybrid_prefill_amd import rag
    plan = synth.rag_plan(R, pool_slots, seed)
    n_cold = len(plan.cold_lengths)
    pool = hp.Pool.allocate(hp.GDN, pool_slots + n_cold, H, d, d, device="cuda")
    for b0 in range(0, pool_slots, 256):                      # untimed pool fill, in batches
        lens = plan.pool_lengths[b0:b0 + 256]
        st = synth.gdn_stream(lens, H, d, d, torch.bfloat16, seed * 1000 + b0, 0.1, "cuda")
        hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, torch.as_tensor(st.seg_offsets).cuda(), pool,
                         torch.arange(b0, b0 + len(lens), dtype=torch.int32, device="cuda"), beta=st.beta)
        del st
    chains, cold_len = rag_chains(plan, R, pool_slots)
    step = rag.plan_step(chains, cold_len)
    sorted_lens = sorted(cold_len.values(), reverse=True)
    cold = synth.gdn_stream(sorted_lens, H, d, d, torch.bfloat16, seed * 1000 + 999, 0.1, "cuda")
    tails = synth.conv_stream((pool_slots + n_cold) * (K - 1), C, torch.bfloat16, seed + 7, "cuda").view(-1, K - 1, C)
    heads = synth.conv_stream((pool_slots + n_cold) * (K - 1), C, torch.bfloat16, seed + 8, "cuda").view(-1, K - 1, C)
    wconv = synth.conv_weights(C, K, seed + 9, "cuda")
    out_S = torch.empty((R, H, d, d), device="cuda")
    conv_out = torch.empty((step.tail_index.numel(), K - 1, C), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    timer = KernelTimer()
    args_ = (step, pool, cold.k, cold.v, cold.beta, cold.log_alpha, tails, heads, wconv, out_S, conv_out)
    mark("rag")
    for _ in range(max(1, args.warmup)):
        rag.prefill_step(*args_, err_flag=err)
    torch.cuda.synchronize()
    n = max(3, args.steps // 4)
    t0 = time.perf_counter()
    for _ in range(n):
        rag.prefill_step(*args_, err_flag=err, timer=timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    assert int(err.item()) == 0 and bool(torch.isfinite(out_S).all())
    b_ms, c_ms, v_ms = timer.mean_ms("build"), timer.mean_ms("compose"), timer.mean_ms("conv")
    ncold_tok = step.n_cold_tokens
    bflops = gdn_build_flops_per_token_head(d, d) * ncold_tok * H
    bbytes = gdn_build_bytes(ncold_tok, H, d, d, n_cold)
    cbytes = compose_bytes([len(c) for c in chains], H, d, d)
    vbytes = conv_bytes(step.tail_index.numel(), C, K)
    prompt_tokens = int(sum(plan.pool_lengths[s] if s < pool_slots else cold_len[s] for c in chains for s in c))
    log(f"rag: {ms:.3f} ms/step; build {b_ms:.3f} ms ({bflops / (b_ms * 1e-3) / 1e12:.0f} TFLOP/s), conv {v_ms:.3f} ms "
        f"({vbytes / (v_ms * 1e-3) / 1e9:.0f} GB/s), compose {c_ms:.3f} ms ({cbytes / (c_ms * 1e-3) / 1e9:.0f} GB/s)")
    del pool, cold
    torch.cuda.empty_cache()
    return {"workload": f"rag_mix_{R}req_pool{pool_slots}_h{H}_d{d}_conv{C}x{K}", "metric": "prompt tokens/s",
            "value": prompt_tokens / (ms * 1e-3), "unit": "tokens/s", "ms": ms,
            "prompt_tokens": prompt_tokens, "cold_tokens": ncold_tok, "cold_segments": n_cold,
            "compositions": step.n_compositions, "boundaries": int(step.tail_index.numel()),
            "kernels": {
                "gdn_build": {"ms": b_ms, "roofline": roofline("mfma", bflops / (b_ms * 1e-3) / 1e12, PEAK_BF16 / 1e12,
                                                                "TFLOP/s", committed_traffic("gdn_build_rag_cold_2584seg")),
                              "hbm_gbps": bbytes / (b_ms * 1e-3) / 1e9},
                "conv_warmup": {"ms": v_ms, "roofline": roofline("hbm", vbytes / (v_ms * 1e-3) / 1e9, PEAK_HBM / 1e9,
                                                                 "GB/s", committed_traffic("conv_warmup_rag_8305x4096_k4"))},
                "compose": {"ms": c_ms, "compositions_per_s": step.n_compositions / (c_ms * 1e-3),
                            "roofline": roofline("hbm", cbytes / (c_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s",
                                                 committed_traffic("gdn_compose_rag_128req"))}}}


def bench_conv_exact(args, R=32, pool_segs=512, H=32, d=128, K=4, seed=601):
    """Conv-coupled exact reuse (conv variant, keys and values from a causal conv over
    C = H (d_k + d_v) raw channels): R requests of 24-96 cached segments (128-1024
    tokens) drawn from a pool whose suffix records were built untimed.  Timed: the
    warmed head keys and values (hypic_conv_kv) and the chains of suffix records with
    the head tokens applied inside the compose (hypic_compose_chain_heads); beside it
    the plain chain of the same records, and the unfused form (a record per head,
    chains of 2m records)."""
    mark("convexact_setup")
    from hybrid_prefill_amd import conv_exact as ce
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(128, 1025, size=pool_segs)
    offs = synth.offsets_from_lengths(lens)
    N, C = int(offs[-1]), H * 2 * d
    c = ce.ConvCache(synth.conv_stream(N, C, torch.bfloat16, seed + 1, "cuda"), offs,
                     synth.write_gate(N, H, seed + 2, "cuda"), synth.gdn_log_decay(N, H, seed + 3, 0.1, "cuda"),
                     synth.conv_weights(C, K, seed + 4, "cuda"), None, 1, H, d, d, torch.bfloat16)
    chains = [rng.integers(0, pool_segs, size=int(m)).astype(np.int32) for m in rng.integers(24, 97, size=R)]
    npos = sum(len(ch) for ch in chains)
    pool = hp.Pool.allocate(hp.GDN, pool_segs + npos, H, d, d, device="cuda")
    ce.cache_segments(c, pool, np.arange(pool_segs))                 # first prefill, untimed
    plan = ce.plan_reuse(c, chains, np.arange(pool_segs), pool_segs)
    out = torch.empty((R, H, d, d), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    plain_offs = torch.as_tensor(np.concatenate([[0], np.cumsum([len(ch) for ch in chains])]).astype(np.int64)).cuda()
    plain_ids = torch.as_tensor(np.concatenate(chains)).cuda()
    mark("convexact")
    for _ in range(max(1, args.warmup)):
        ce.reuse(c, plan, pool, out_S=out, err_flag=err)
    torch.cuda.synchronize()
    timer = KernelTimer()
    n = max(3, args.steps // 4)
    t0 = time.perf_counter()
    for _ in range(n):
        ce.reuse(c, plan, pool, out_S=out, err_flag=err, timer=timer)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    assert int(err.item()) == 0 and bool(torch.isfinite(out).all())
    (plain_ms,) = kernel_pass((("plain", lambda: hp.compose_chain(pool, plain_offs, plain_ids, out_S=out)),), n)
    prompt_tokens = int(sum(int(lens[s]) for ch in chains for s in ch))
    parts = {k_: timer.mean_ms(k_) for k_ in ("conv_kv", "compose")}
    # the unfused form for comparison: a record per head, chains of 2m records
    timer2 = KernelTimer()
    for _ in range(n):
        ce.reuse(c, plan, pool, out_S=out, err_flag=err, timer=timer2, fused=False)
    torch.cuda.synchronize()
    unfused = {k_: timer2.mean_ms(k_) for k_ in ("conv_kv", "head_build", "compose")}
    log(f"conv exact: {ms:.3f} ms/step (conv_kv {parts['conv_kv']:.3f}, compose with head tokens "
        f"{parts['compose']:.3f} ms); plain chain {plain_ms:.3f} ms; with head records instead: conv_kv "
        f"{unfused['conv_kv']:.3f}, head records {unfused['head_build']:.3f}, compose of {2 * npos} records "
        f"{unfused['compose']:.3f} ms")
    del pool, c
    torch.cuda.empty_cache()
    return {"workload": f"conv_exact_reuse_{R}req_pool{pool_segs}_h{H}_d{d}_conv{C}x{K}",
            "metric": "prompt tokens/s", "value": prompt_tokens / (ms * 1e-3), "unit": "tokens/s", "ms": ms,
            "head_tokens": int(plan.head_src.numel()), "records_composed": npos,
            "kernels_ms": parts, "plain_chain_ms": plain_ms, "head_records_path_ms": unfused}


def bench_kda(args, H=16, d=128, nseg=8, seg_len=2048, seed=701):
    """KDA family (A_t = (I - beta k k^T) diag(alpha_t), per-channel gates), H=16, d=128,
    bf16, 8 x 2048 tokens (the scalar / diagonal workload's shape): build of every
    record (T_C, S) and the 8-segment chain.  The build is the chunked kernel on the
    fp32 matrix cores; its roofline counts the definition's 5 d_k (d_k + d_v) FLOP per
    token-head against the fp32 matrix peak."""
    mark("kda")
    N = nseg * seg_len
    k = synth.keys(N, H, d, torch.bfloat16, seed, "cuda")
    v = synth.values(N, H, d, torch.bfloat16, seed + 1, "cuda")
    b = synth.write_gate(N, H, seed + 2, "cuda")
    la = synth.diagonal_log_gates(N, H, d, seed + 3, 16.0, "cuda")
    offs = torch.as_tensor(synth.even_offsets(nseg, seg_len)).cuda()
    slots = torch.arange(nseg, dtype=torch.int32, device="cuda")
    chain = torch.tensor([0, nseg], dtype=torch.int64, device="cuda")
    pool = hp.Pool.allocate(hp.KDA, nseg, H, d, d, device="cuda")
    for _ in range(max(1, args.warmup)):
        hp.build_segment(hp.KDA, k, v, la, offs, pool, slots, beta=b)
    torch.cuda.synchronize()
    b_ms, c_ms = kernel_pass((("build", lambda: hp.build_segment(hp.KDA, k, v, la, offs, pool, slots, beta=b)),
                              ("compose", lambda: hp.compose_chain(pool, chain, slots))), max(3, args.steps // 4))
    flops = 5.0 * d * (d + d) * N * H
    log(f"kda: build {b_ms:.3f} ms ({flops / (b_ms * 1e-3) / 1e12:.2f} TFLOP/s fp32), compose {c_ms:.3f} ms")
    del pool
    torch.cuda.empty_cache()
    return {"workload": f"kda_build_h{H}_d{d}_{nseg}x{seg_len}", "metric": "tokens/s", "value": N / (b_ms * 1e-3),
            "unit": "tokens/s", "ms": b_ms, "compose_ms": c_ms,
            "roofline": roofline("mfma", flops / (b_ms * 1e-3) / 1e12, PEAK_FP32 / 1e12, "TFLOP/s")}


def hbm_attainable(gib=4):
    """Context for the HBM fractions: the rate PyTorch's own device copy (read + write)
    reaches on this GPU over `gib` GiB."""
    x = torch.empty((gib << 28,), dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    (ms,) = kernel_pass((("copy", lambda: y.copy_(x)),), 5)
    out = {"copy_gbps": 2 * x.numel() * 4 / (ms * 1e-3) / 1e9}
    del x, y
    torch.cuda.empty_cache()
    log(f"attainable: torch copy {out['copy_gbps']:.0f} GB/s (read + write)")
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seg_len=2048, H=32, d=128, nseg_sample=16, seed=301):
    """fp64 oracle on the host: build of nseg_sample of the main workload's 16
    segments, all heads (the first nseg_sample segments' tokens, same seed), on all
    of the host's OpenMP threads; beside it smaller samples on one thread and a
    compose sample (see cpu_detail)."""
    import oracle
    st = synth.gdn_stream([seg_len] * nseg_sample, H, d, d, torch.bfloat16, seed, 0.1, "cpu")
    k, v = st.k.double().numpy(), st.v.double().numpy()
    b, la = st.beta.double().numpy(), st.log_alpha.double().numpy()
    t0 = time.perf_counter()
    oracle.build_segments(oracle.GDN, k, v, la, st.seg_offsets, beta=b)
    dt = time.perf_counter() - t0
    toks = seg_len * nseg_sample
    del k, v, b, la, st
    return {"value": toks / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"GDN build of {nseg_sample} x {seg_len}-token segment(s) x {H} heads, d={d}, "
                      f"fp64 token-by-token recurrence ({dt:.1f} s wall on {oracle.num_threads()} threads)",
            "detail": cpu_detail()}


def cpu_detail(seed=901):
    """Oracle samples of the other workloads: one thread (the build of the small GDN
    workload, one 2048-token segment of the scalar and of the diagonal workload, one
    32-record chain of the pool compose) and all threads (8 chains of the pool compose)."""
    import oracle
    out = {}
    nthreads = oracle.num_threads()
    rng = np.random.default_rng(seed)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def records(nslots, H, dk, dv):
        q, _ = np.linalg.qr(rng.standard_normal((nslots, H, dk, dk)))
        return (rng.uniform(-0.5, 0.0, size=(nslots, H)), 0.9 * q, rng.standard_normal((nslots, H, dk, dv)))

    try:
        oracle.set_num_threads(1)
        st = synth.gdn_stream([256, 256], 1, 64, 64, torch.float32, 101, 0.1, "cpu")
        dt = timed(lambda: oracle.build_segments(oracle.GDN, st.k.double().numpy(), st.v.double().numpy(),
                                                 st.log_alpha.double().numpy(), st.seg_offsets,
                                                 beta=st.beta.double().numpy()))
        out["gdn_h1_d64_fp32_2x256_build_1thread"] = {"value": 512 / dt, "unit": "tokens/s", "s": dt}
        N, H, D = 2048, 16, 128
        k = synth.keys(N, H, D, torch.bfloat16, 2011, "cpu").double().numpy()
        v = synth.values(N, H, D, torch.bfloat16, 2012, "cpu").double().numpy()
        lg = synth.scalar_log_gamma(H, 2014, device="cpu").double().numpy()
        dt = timed(lambda: oracle.build_segments(oracle.SCALAR, k, v, np.broadcast_to(lg, (N, H)).copy(), [0, N]))
        out["scalar_h16_d128_1x2048_build_1thread"] = {"value": N / dt, "unit": "tokens/s", "s": dt}
        lgd = synth.diagonal_log_gates(N, H, D, 2014, device="cpu").double().numpy()
        dt = timed(lambda: oracle.build_segments(oracle.DIAGONAL, k, v, lgd, [0, N]))
        out["diagonal_h16_d128_1x2048_build_1thread"] = {"value": N / dt, "unit": "tokens/s", "s": dt}
        del k, v, lgd
        ell, P, S = records(32, 32, 128, 128)
        ids = np.arange(32, dtype=np.int32)
        dt = timed(lambda: oracle.compose(oracle.GDN, ell, P, S, [0, 32], ids))
        out["gdn_compose_h32_d128_1x32_1thread"] = {"value": 32 / dt, "unit": "compositions/s", "s": dt,
                                                    "note": "all 32 heads per composition, as the GPU counts"}
    finally:
        oracle.set_num_threads(nthreads)
    ids = rng.integers(0, 32, size=8 * 32).astype(np.int32)
    dt = timed(lambda: oracle.compose(oracle.GDN, ell, P, S, np.arange(0, 8 * 32 + 1, 32), ids))
    out["gdn_compose_h32_d128_8x32"] = {"value": 8 * 32 / dt, "unit": "compositions/s", "s": dt,
                                        "threads": nthreads}
    log("cpu detail: " + ", ".join(f"{k_} {v_['value']:.3g} {v_['unit']}" for k_, v_ in out.items()))
    return out


def measured_peaks():
    """What this machine delivers: a streaming read of 4 GiB (16384 workgroups of 512
    threads, non-temporal 16-byte loads: the best of a sweep over grid sizes, unroll
    depths and cache policies), a streaming copy of 1 GiB with the same loads and
    non-temporal stores (the rate of a kernel that writes as much as it reads), and a
    loop of bf16 32x32x16 matrix-core products on every SIMD (libhypic_peaks.so)."""
    mark("peaks")
    L = peaks_lib()
    stream = torch.cuda.current_stream().cuda_stream
    buf = torch.empty(1 << 30, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    nbytes = buf.numel() * 4
    cbytes = dst.numel() * 4                      # 1 GiB read and 1 GiB written
    blocks = 256 * 64
    rd = lambda: L.hypic_peak_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream)
    cp = lambda: L.hypic_peak_copy(buf.data_ptr(), dst.data_ptr(), cbytes, blocks, stream)
    iters, mblocks = 512, 256 * 4
    mf = lambda: L.hypic_peak_mfma(iters, mblocks, sink.data_ptr(), stream)
    for _ in range(2):
        assert rd() == 0 and mf() == 0 and cp() == 0
    ks = launch_stats((("read", rd), ("copy", cp), ("mfma", mf)), 8)
    flop = iters * 4 * 32768.0 * mblocks * 4
    out = {"read_gbps": nbytes / (ks["read"]["p50"] * 1e-3) / 1e9, "read_ms": ks["read"],
           "copy_gbps": 2 * cbytes / (ks["copy"]["p50"] * 1e-3) / 1e9, "copy_ms": ks["copy"],
           "bf16_mfma_tflops": flop / (ks["mfma"]["p50"] * 1e-3) / 1e12, "mfma_ms": ks["mfma"]}
    del buf, dst, sink
    torch.cuda.empty_cache()
    log(f"measured peaks: read {out['read_gbps']:.0f} GB/s, copy {out['copy_gbps']:.0f} GB/s (read + write), "
        f"bf16 MFMA {out['bf16_mfma_tflops']:.0f} TFLOP/s")
    return out


def algorithmic_bytes(key):
    """Algorithmic HBM bytes per launch of a TRAFFIC_KERNELS entry (the RAG mix's
    sizes come from its seeded plan, rebuilt on the host)."""
    N, H, d = 16 * 2048, 32, 128
    table = {
        "gdn_build_h32_d128_16x2048": lambda: gdn_build_bytes(N, H, d, d, 16),
        "gdn_compose_h32_d128_chain16": lambda: compose_bytes([16], H, d, d),
        "gdn_forward_h32_d128_16x2048": lambda: forward_bytes(N, H, d, d, 16),
        "gdn_forward_records_h32_d128_16x2048": lambda: forward_bytes(N, H, d, d, 16, records=True),
        "gdn_compose_pool4096_h32_d128_64x32": lambda: compose_bytes([32] * 64, H, d, d),
        "scalar_build_h16_d128_8x2048": lambda: sd_build_bytes(hp.SCALAR, 8 * 2048, 16, d, d, 8),
        "diagonal_build_h16_d128_8x2048": lambda: sd_build_bytes(hp.DIAGONAL, 8 * 2048, 16, d, d, 8),
        "conv_warmup_rag_8305x4096_k4": lambda: conv_bytes(8305, 4096, 4),
    }
    if key in table:
        return table[key]()
    if key in ("gdn_build_rag_cold_2584seg", "gdn_compose_rag_128req"):
        from hybrid_prefill_amd import rag
        R, pool_slots = 128, 4096
        chains, cold_len = rag_chains(synth.rag_plan(R, pool_slots, 501), R, pool_slots)
        step = rag.plan_step(chains, cold_len, device="cpu")
        if key.startswith("gdn_build"):
            return gdn_build_bytes(step.n_cold_tokens, H, d, d, len(cold_len))
        return compose_bytes([len(c) for c in chains], H, d, d)
    return None


COUNTER_RUN = ("python $REPO/bench.py --steps 2 --warmup 1 --no-cpu --calib-copy")


def summarize_traffic(fetch_csv, write_csv, out_dir):
    """Turn two rocprofv3 --pmc runs of the benchmark (FETCH_SIZE, then WRITE_SIZE, with
    --calib-copy) into one committed summary per timed kernel: each counter scaled by
    what it reads for the 1 GiB device copy in the same process (the process's first
    copy), the median over that kernel's launches at its grid, and the hash of its
    sources."""
    def load(path):
        return sorted(((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
                       for r in csv.DictReader(open(path))), key=lambda t: t[0])

    F, W = load(fetch_csv), load(write_csv)
    phase_f, phase_w = dispatch_phases(F), dispatch_phases(W)

    def first_copy(rows):
        return next(v for _, n, g, v in rows if "__amd_rocclr_copyBuffer" in n and g == 131072)

    def per_launch(rows, phases, frag, grid, phase):
        vals = [v for d, n, g, v in rows
                if frag in n and (grid is None or g == grid) and phases.get(d, "marker") == phase]
        return (float(np.median(vals)) if vals else None), len(vals)

    copy_bytes = float(1 << 30)
    f_copy, w_copy = first_copy(F), first_copy(W)
    sf, sw = copy_bytes / (f_copy * 1024), copy_bytes / (w_copy * 1024)
    for key, (frag, grid, phase, sources, title) in TRAFFIC_KERNELS.items():
        f_k, nf = per_launch(F, phase_f, frag, grid, phase)
        w_k, nw = per_launch(W, phase_w, frag, grid, phase)
        if f_k is None or w_k is None:
            log(f"summarize-traffic: no launches of {frag} (grid {grid}, phase {phase}); {key} skipped")
            continue
        rd, wr = f_k * 1024 * sf, w_k * 1024 * sw
        alg = algorithmic_bytes(key)
        lines = [f"# HBM traffic -- {title}", "",
                 "Two rocprofv3 passes over the benchmark (all legs, no CPU leg), one counter each, with one "
                 "untimed 1 GiB device copy first as calibration:", "",
                 "```",
                 "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv "
                 f"-d $REPO/gpurun_out/pmc_fetch -o fetch -- {COUNTER_RUN}",
                 "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv "
                 f"-d $REPO/gpurun_out/pmc_write -o write -- {COUNTER_RUN}",
                 "python $REPO/bench.py --summarize-traffic $REPO/gpurun_out/pmc_fetch/fetch_counter_collection.csv "
                 "$REPO/gpurun_out/pmc_write/write_counter_collection.csv $REPO/profiles",
                 "```", "",
                 f"Kernel `{frag.rstrip('(')}`" + (f", grid {grid} threads" if grid else "")
                 + f", launches of the bench's `{phase}` phase.", "",
                 "| counter | copy kernel (KiB) | copy bytes (KiB) | scale | kernel per launch (KiB, median) "
                 "| launches | scaled |",
                 "|---|---|---|---|---|---|---|",
                 f"| FETCH_SIZE | {f_copy:.0f} | {copy_bytes / 1024:.0f} | {sf:.3f} | {f_k:.0f} | {nf} | "
                 f"{rd / 1e6:.1f} MB |",
                 f"| WRITE_SIZE | {w_copy:.0f} | {copy_bytes / 1024:.0f} | {sw:.3f} | {w_k:.0f} | {nw} | "
                 f"{wr / 1e6:.1f} MB |",
                 "",
                 f"HBM bytes per launch: {(rd + wr) / 1e6:.1f} MB"
                 + (f" (algorithmic {alg / 1e6:.1f} MB: {(rd + wr) / alg:.2f}x)" if alg else ""),
                 "",
                 f"kernel source sha256[:16]: `{source_sha(sources)}` ({', '.join(sources)})", ""]
        with open(os.path.join(out_dir, f"{key}_traffic.md"), "w") as f:
            f.write("\n".join(lines))
        print(f"{key}: {(rd + wr) / 1e6:.1f} MB per launch" + (f" ({(rd + wr) / alg:.2f}x algorithmic)" if alg else ""))


MFMA_KERNELS = (
    # (kernel name fragment, grid in threads (None: any), bench phase, workload, MOPS type)
    ("gdn_build_mfma_kernel(", None, "main", "GDN build, main workload", "BF16"),
    ("gdn_build_mfma_kernel(", None, "rag", "GDN build, RAG mix cold segments", "BF16"),
    ("gdn_chunk_mfma_kernel<false, true>", 262144, "forward", "GDN prefill forward, outputs only", "BF16"),
    ("gdn_chunk_mfma_kernel<true, true>", 393216, "forward", "GDN prefill forward with records", "BF16"),
    ("compose_sliced_mfma_kernel", 65536, "main", "GDN compose, 16-segment chain", "BF16"),
    ("compose_dense_mfma_kernel<false, false>", 524288, "compose", "GDN compose, 4096-slot pool", "BF16"),
    ("sd_build_mfma_kernel<0, 2>", 131072, "sd", "scalar build", "BF16"),
    ("sd_build_mfma_kernel<1, 2>", 196608, "sd", "diagonal build", "BF16"),
    ("kda_chunk_mfma_kernel", 131072, "kda", "KDA build (fp32 matrix cores)", "F32"),
)


def summarize_mfma(csv_path, out_md):
    """Matrix-core utilisation per kernel from one rocprofv3 --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
    SQ_INSTS_VALU_MFMA_MOPS_F32: busy fraction = busy cycles summed over the 1024
    SIMDs / (1024 x GPU-active cycles per XCD); clock = GPU-active cycles per XCD
    over the launch's duration; executed FLOP = MOPS x 512."""
    disp = {}
    for r in csv.DictReader(open(csv_path)):
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                    "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    phases = dispatch_phases([(k, d["name"], d["grid"]) for k, d in disp.items()])
    lines = ["# Matrix-core utilisation per kernel (bench workloads)", "",
             "One rocprofv3 counter pass over the benchmark (all legs, no CPU leg):", "",
             "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 --output-format csv -d $REPO/gpurun_out/pmc_mfma "
             "-o mfma -- python $REPO/bench.py --steps 2 --warmup 1 --no-cpu",
             "python $REPO/bench.py --summarize-mfma $REPO/gpurun_out/pmc_mfma/mfma_counter_collection.csv <this file>",
             "```", "",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); clock = "
             "(GRBM_GUI_ACTIVE / 8) / duration; executed TFLOP/s = MOPS x 512 / duration (counted at the "
             "profiled launch's duration). For launches of a few tens of µs the GPU-active count also covers the "
             "dispatch's set-up and drain, so their clock reads high.", "",
             "| kernel | workload | grid | launches | µs (median) | clock GHz | MFMA busy | executed TFLOP/s | MOPS type |",
             "|---|---|---|---|---|---|---|---|---|"]
    for frag, grid, phase, title, ty in MFMA_KERNELS:
        ds = [d for k, d in disp.items() if frag in d["name"] and (grid is None or d["grid"] == grid)
              and phases.get(k, "marker") == phase and "GRBM_GUI_ACTIVE" in d]
        if not ds:
            continue
        grid = ds[0]["grid"]
        dur = float(np.median([d["dur"] for d in ds])) * 1e-9
        grbm = float(np.median([d["GRBM_GUI_ACTIVE"] for d in ds])) / 8
        busy = float(np.median([d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds])) / (1024 * grbm)
        mops = float(np.median([d.get(f"SQ_INSTS_VALU_MFMA_MOPS_{ty}", 0.0) for d in ds]))
        lines.append(f"| `{frag.rstrip('(')}` | {title} | {grid} | {len(ds)} | {dur * 1e6:.1f} | "
                     f"{grbm / dur / 1e9:.2f} | {busy:.3f} | {mops * 512 / dur / 1e12:.1f} | {ty} |")
    lines.append("")
    srcs = sorted({n for v in TRAFFIC_KERNELS.values() for n in v[3]} | {"build_kda_mfma.hip"})
    lines.append(f"sources sha256[:16]: `{source_sha(srcs)}` ({', '.join(srcs)})")
    lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


TRACE_WORKLOADS = {
    # (kernel name as shown, x extent of the grid in threads (None: any), bench phase) -> workload
    ("compose_dense_mfma_kernel<false, false>", 262144, "convexact"):
        "GDN compose, conv-exact reuse (unfused leg, and the plain chain over the suffix records)",
    ("compose_dense_mfma_kernel<false, false>", 524288, "compose"): "GDN compose, 4096-slot pool, 64 requests x 32 slots",
    ("compose_dense_mfma_kernel<false, false>", 1048576, "rag"): "GDN compose, RAG mix, 128 requests x 24-96 slots",
    ("compose_dense_mfma_kernel<false, true>", 262144, "convexact"):
        "GDN compose with warmed head tokens (conv-exact reuse, 32 requests, 5631 head tokens)",
    ("compose_sd_wide_kernel<0, 128, 128>", 65536, "sd"): "scalar compose, 8-segment chain, H=16",
    ("compose_sd_wide_kernel<1, 128, 128>", 65536, "sd"): "diagonal compose, 8-segment chain, H=16",
    ("compose_sliced_mfma_kernel", 32768, "kda"): "KDA compose, 8-segment chain, H=16 (four column slices)",
    ("compose_sliced_mfma_kernel", 65536, "main"): "GDN compose, 16-segment chain, H=32, 4 column slices (main step)",
    ("conv_kv_kernel", None, "convexact"): "conv_kv, conv-exact reuse head tokens",
    ("conv_kv_kernel", None, "convexact_setup"): "conv_kv, conv-exact suffix records (untimed setup)",
    ("conv_warmup_vec_kernel<unsigned short, 4>", None, "rag"):
        "conv warm-up, RAG mix, 8305 boundaries x 4096 channels, kernel 4",
    ("gdn_build_mfma_kernel", None, "main"): "GDN build, H=32, d=128, bf16, 16 x 2048 tokens (main step)",
    ("gdn_build_mfma_kernel", None, "compose_setup"): "GDN build, 4096 x 64-token pool fill (untimed setup)",
    ("gdn_build_mfma_kernel", None, "rag_setup"): "GDN build, RAG pool fill batches of 256 segments (untimed setup)",
    ("gdn_build_mfma_kernel", None, "rag"): "GDN build, RAG mix cold segments (2584 x 32 heads)",
    ("gdn_build_mfma_kernel", None, "convexact_setup"): "GDN build, conv-exact suffix records (untimed setup)",
    ("gdn_build_mfma_kernel", None, "convexact"): "GDN build, conv-exact head records (unfused leg)",
    ("gdn_chunk_mfma_kernel<false, true>", 262144, "forward"):
        "GDN prefill forward, outputs only, H=32, d=128, bf16, 16 x 2048 tokens",
    ("gdn_chunk_mfma_kernel<true, true>", 393216, "forward"):
        "GDN prefill forward with the records as side-outputs, same workload",
    ("kda_chunk_mfma_kernel<unsigned short>", 131072, "kda"):
        "KDA build, H=16, d=128, bf16, 8 x 2048 tokens (chunk form, fp32 MFMA, two roles)",
    ("sd_build_mfma_kernel<0, 2>", 131072, "sd"): "scalar build, H=16, d=128, bf16, 8 x 2048 tokens",
    ("sd_build_mfma_kernel<1, 2>", 196608, "sd"): "diagonal build, H=16, d=128, bf16, 8 x 2048 tokens",
    ("peak_mfma_kernel", 262144, "peaks"): "measured-peak bf16 MFMA loop, 1024 x 4 waves x 512 x 4 products",
    ("peak_read_kernel", 8388608, "peaks"): "measured-peak streaming read of 4 GiB",
    ("peak_copy_kernel", 8388608, "peaks"): "measured-peak streaming copy of 1 GiB (1 GiB read, 1 GiB written)",
}


def _trace_workload(short, grid, phase):
    """The TRACE_WORKLOADS key of a dispatch, or None."""
    for g in (grid, None):
        if (short, g, phase) in TRACE_WORKLOADS:
            return (short, g, phase)
    return None


def _short_kernel_name(name):
    """'void hypic::(anonymous namespace)::k<a, b>(hypic::Args)' -> 'k<a, b>'."""
    n = name[5:] if name.startswith("void ") else name
    for pre in ("hypic::(anonymous namespace)::", "(anonymous namespace)::"):
        n = n.replace(pre, "")
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):                     # drop the parameter list at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return n[:cut]


def _trace_key(short):
    if short.startswith("conv_kv_kernel"):
        return "conv_kv_kernel"                    # its template arguments demangle differently by run
    return short


def summarize_trace(trace_csv, stats_csv, bench_json, out_md):
    """The kernel-trace summary of the library's kernels: per (kernel, grid) launch
    durations from rocprofv3's kernel trace, rocprofv3's own --stats table, and the
    benchmark's HIP-event figures of an unprofiled run for comparison."""
    groups = {}
    rows = list(csv.DictReader(open(trace_csv)))
    phases = dispatch_phases([(int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size_X"])) for r in rows])
    for r in rows:
        short = _short_kernel_name(r["Kernel_Name"])
        grid = int(r["Grid_Size_X"])
        wk = _trace_workload(_trace_key(short), grid, phases.get(int(r["Dispatch_Id"]), "marker"))
        if wk is None:
            continue
        g = groups.setdefault((wk[0], grid, wk[2], short), {"dur": [], "row": r, "wk": wk})
        g["dur"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = ["# rocprofv3 kernel trace -- library kernels, per launch shape", "",
             "Command (repo at $REPO on the MI355X box; the default bench run without the CPU leg):", "",
             "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $REPO/gpurun_out/prof_all -o all -- python $REPO/bench.py --no-cpu",
             "python $REPO/bench.py --summarize-trace $REPO/gpurun_out/prof_all/all_kernel_trace.csv "
             "$REPO/gpurun_out/prof_all/all_kernel_stats.csv BENCH_JSON <this file>",
             "```", "",
             "Durations are per launch (End - Start of the kernel trace), grouped by kernel, grid and bench "
             "phase; \"grid\" is the x extent in threads (the conv warm-up grid is 512 x 8305, boundaries on y). "
             "The GDN build runs the same grid for every workload of more than a few hundred (segment, head) "
             "units, so launches are attributed to the bench phase whose marker launch precedes them (a "
             "16-byte `peak_copy_kernel` with as many workgroups as the phase's number). The `peak_*` "
             "kernels are the measured-peak microbenchmarks (libhypic_peaks.so). conv_kv's template arguments "
             "demangle garbled in the profiler.", "",
             "| kernel | grid (threads) | phase | wg | LDS B | VGPR | AGPR | launches | mean µs | min µs | workload |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(groups, key=lambda k: (k[0].startswith("peak_"), k[0], k[1], k[2])):
        g = groups[key]
        r, d = g["row"], g["dur"]
        lines.append(f"| `{key[3]}` | {key[1]} | {key[2]} | {r['Workgroup_Size_X']} | {r['LDS_Block_Size']} | "
                     f"{r['VGPR_Count']} | {r['Accum_VGPR_Count']} | {len(d)} | {np.mean(d):.1f} | {np.min(d):.1f} | "
                     f"{TRACE_WORKLOADS[g['wk']]} |")
    lines += ["", "rocprofv3's own `--stats` summary (`all_kernel_stats.csv`) for the same run, all launches of a "
              "kernel together:", "", "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        short = _short_kernel_name(r["Name"])
        if not any(_trace_key(short) == k[0] for k in TRACE_WORKLOADS):
            continue
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) * 1e-3:.1f} | "
                     f"{float(r['MinNs']) * 1e-3:.1f} | {float(r['MaxNs']) * 1e-3:.1f} |")
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    k, sec = b["kernels"], {s["workload"]: s for s in b.get("secondary", [])}
    gb = k["gdn_build"]["ms_stats"]
    parts = [f"GDN build {gb['mean'] * 1e3:.0f} µs (main step; p10 {gb['p10'] * 1e3:.0f}, p90 {gb['p90'] * 1e3:.0f})",
             f"main-step compose {k['gdn_compose_chain16']['ms'] * 1e3:.0f} µs"]
    for name, label in (("gdn_prefill_forward_h32_d128_bf16_16x2048", "prefill forward"),
                        ("gdn_compose_pool4096_h32_d128_64x32", "pool compose"),
                        ("scalar_build_h16_d128_8x2048", "scalar build"),
                        ("diagonal_build_h16_d128_8x2048", "diagonal build"),
                        ("kda_build_h16_d128_8x2048", "KDA build")):
        s = sec.get(name)
        if s is None:
            continue
        if "with_records" in s:
            parts.append(f"{label} {s['ms'] * 1e3:.0f} µs (outputs only) and {s['with_records']['ms'] * 1e3:.0f} µs "
                         "(with records)")
        else:
            parts.append(f"{label} {s['ms'] * 1e3:.0f} µs")
    mp = b.get("measured_peaks") or {}
    if mp:
        if "copy_gbps" in mp:
            parts.append(f"streaming copy of 1 GiB {mp['copy_gbps'] / 1e3:.2f} TB/s (read + write)")
        parts.append(f"streaming read of 4 GiB {mp['read_gbps'] / 1e3:.2f} TB/s, bf16 MFMA loop "
                     f"{mp['bf16_mfma_tflops'] / 1e3:.2f} PFLOP/s")
    lines += ["", "The bench's own HIP-event figures (mean over the timed launches) for the same kernels in the "
              "unprofiled run of the same build:", ", ".join(parts) + ".", ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "main", "forward", "sd", "compose", "rag", "convexact", "kda", "peaks"],
                    default="all", help="main: only the headline GDN step; otherwise it plus that leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one untimed 1 GiB device copy (reference kernel for HBM byte counters)")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_DIR"),
                    help="write the HBM-traffic summaries of the timed kernels from two rocprofv3 counter runs")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("CSV", "OUT_MD"),
                    help="write the matrix-core utilisation summary from one rocprofv3 counter run")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_CSV", "STATS_CSV", "BENCH_JSON", "OUT_MD"),
                    help="write the kernel-trace summary from one rocprofv3 kernel-trace run and a bench line")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 (the path shards by "
              "(segment, head) with no collective, see the design notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    hp.lib()
    torch.cuda.synchronize()
    if args.calib_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step, N, kern, flops, b_ms, w = bench_main(args)
    ms_eager = w["ms_eager"]
    traffic = committed_traffic()
    secondary = []
    if args.only in ("all", "forward"):
        secondary.append(bench_forward(args, w, b_ms))
    del w
    torch.cuda.empty_cache()
    if args.only in ("all", "compose"):
        secondary.append(bench_compose_pool(args))
    if args.only in ("all", "sd"):
        secondary.extend(bench_sd(args))
    if args.only in ("all", "rag"):
        secondary.append(bench_rag(args))
    if args.only in ("all", "convexact"):
        secondary.append(bench_conv_exact(args))
    if args.only in ("all", "kda"):
        secondary.append(bench_kda(args))
    attainable = hbm_attainable()
    peaks = measured_peaks() if args.only in ("all", "peaks", "main") else None
    cpu = None if args.no_cpu else cpu_baseline()
    achieved = flops / (b_ms * 1e-3) / 1e12
    if peaks:
        peaks["gdn_build_frac_of_measured_mfma"] = achieved / peaks["bf16_mfma_tflops"]
    line = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gdn_build_compose_h32_d128_bf16_16x2048",
                   "heads": 32, "d_k": 128, "d_v": 128, "segments": 16, "segment_tokens": 2048,
                   "kv_dtype": "bf16", "record_dtype": "fp32", "parallelism": "none (1 GPU)",
                   "step_launch": "hip graph replay"},
        "ms_per_step_eager_launches": ms_eager,
        "roofline": roofline("mfma", achieved, PEAK_BF16 / 1e12, "TFLOP/s", traffic),
        "cpu_baseline": cpu,
        "kernels": kern,
        "secondary": secondary,
        "hbm_attainable": attainable,
        "measured_peaks": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
