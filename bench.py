"""Benchmark of the HYPIC linear-layer hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  main workload  GDN, H=32, d_k=d_v=128, bf16 k/v, fp32 records: one 32768-token
                 request split into 16 segments of 2048 tokens; build all 512
                 (segment, head) records, then compose the 16-segment chain to
                 the request's final state.
Secondary lines (same JSON object, key "secondary"):
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

Inputs are resident in HBM before the timed region starts.  Kernel durations
come from HIP events recorded on the stream the kernels are launched on.
The cpu_baseline leg times the fp64 oracle on a bounded sample on the host.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only main|sd|compose|rag|convexact|kda] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
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
# HBM bytes per launch of the GDN build kernel, from rocprofv3 FETCH_SIZE + WRITE_SIZE
# (scaled by the copy-kernel calibration); None until measured for the current kernel.
# HBM bytes per launch of the GDN build on the main workload (rocprofv3 FETCH_SIZE and
# WRITE_SIZE, each scaled by what the counter reads for a copy of known size: read
# 604.4 MB + write 67.1 MB); None whenever the kernel changed since the counters were taken
TRAFFIC_GDN_BUILD = 671.5e6


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


def kernel_pass(launches, n):
    """Mean duration of each launch in `launches` (name -> callable, idempotent): one
    HIP-event pair around n back-to-back launches of it on the current stream, so the
    per-launch event overhead is spread over n; a short device spin first lets the
    host run ahead, so host time is never counted as kernel time."""
    out = []
    for name, fn in launches:
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(5e6))
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / n)
    return tuple(out)


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


def bench_main(args):
    w = gdn_workload()
    for _ in range(args.warmup):
        gdn_step(w)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gdn_step(w)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(w["err"].item()) == 0
    ms_step = wall * 1e3 / args.steps
    # per-kernel durations: the same steps again with the launch queue filled ahead
    # (a short device spin first), so that host time between an event and its launch
    # never shows up as kernel time
    st_, pool_ = w["st"], w["pool"]
    b_ms, c_ms = kernel_pass((
        ("build", lambda: hp.build_segment(hp.GDN, st_.k, st_.v, st_.log_alpha, w["offs"], pool_, w["slots"],
                                           beta=st_.beta, err_flag=w["err"])),
        ("compose", lambda: hp.compose_chain(pool_, w["chain_offs"], w["slots"], out_S=w["out_S"],
                                             err_flag=w["err"]))), args.steps)
    N, H, dk, dv, nseg = w["N"], w["H"], w["dk"], w["dv"], w["nseg"]
    flops = gdn_build_flops_per_token_head(dk, dv) * N * H
    bbytes = gdn_build_bytes(N, H, dk, dv, nseg)
    cbytes = compose_bytes([nseg], H, dk, dv)
    log(f"main: {ms_step:.3f} ms/step wall; build {b_ms:.3f} ms, compose {c_ms:.3f} ms; "
        f"build {flops / (b_ms * 1e-3) / 1e12:.1f} TFLOP/s, {bbytes / (b_ms * 1e-3) / 1e9:.0f} GB/s")
    kern = {
        "gdn_build": {"ms": b_ms, "algorithmic_flop": flops, "algorithmic_bytes": bbytes,
                      "tflops": flops / (b_ms * 1e-3) / 1e12, "gbps": bbytes / (b_ms * 1e-3) / 1e9,
                      "tokens_per_s": N / (b_ms * 1e-3)},
        "gdn_compose_chain16": {"ms": c_ms, "algorithmic_bytes": cbytes, "gbps": cbytes / (c_ms * 1e-3) / 1e9,
                                "compositions_per_s": nseg / (c_ms * 1e-3)},
    }
    del w
    torch.cuda.empty_cache()
    return ms_step, N, kern, flops, b_ms


def bench_compose_pool(args, slots=4096, H=32, d=128, R=64, m=32, seg_len=64, seed=401):
    """Pool of GDN records (filled untimed by the build), R requests x m slot ids."""
    st = synth.gdn_stream([seg_len] * slots, H, d, d, torch.bfloat16, seed, 0.01, "cuda")
    pool = hp.Pool.allocate(hp.GDN, slots, H, d, d, device="cuda")
    hp.build_segment(hp.GDN, st.k, st.v, st.log_alpha, torch.as_tensor(st.seg_offsets).cuda(), pool,
                     torch.arange(slots, dtype=torch.int32, device="cuda"), beta=st.beta)
    del st
    torch.cuda.synchronize()
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
            "roofline": roofline("hbm", nbytes / (ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s")}


def bench_sd(args, H=16, d=128, nseg=8, seg_len=2048, seed=201, copies=3):
    """Scalar and diagonal builds + their 8-segment chains.  The inputs are
    rotated over `copies` seeded copies so that the timed working set exceeds
    the 256 MB Infinity Cache (one copy of k, v and the gates would fit)."""
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
                    "roofline": roofline("hbm", nb / (b_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s")})
        del las, pool
    return out


def conv_bytes(B, C, K, x_bytes=2):
    return B * (2 * (K - 1) * C * x_bytes + (K - 1) * C * 4) + C * K * 4


def bench_rag(args, R=128, pool_slots=4096, H=32, d=128, C=4096, K=4, seed=501):
    """RAG-shaped step: 128 requests of 24-96 segments (128-1024 tokens), 70 %
    cache hits from a 4096-slot pool built untimed, 30 % cold segments built in
    the step, conv warm-up at every boundary, all chains composed."""
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
                                                                "TFLOP/s")},
                "conv_warmup": {"ms": v_ms, "roofline": roofline("hbm", vbytes / (v_ms * 1e-3) / 1e9, PEAK_HBM / 1e9,
                                                                 "GB/s")},
                "compose": {"ms": c_ms, "compositions_per_s": step.n_compositions / (c_ms * 1e-3),
                            "roofline": roofline("hbm", cbytes / (c_ms * 1e-3) / 1e9, PEAK_HBM / 1e9, "GB/s")}}}


def bench_conv_exact(args, R=32, pool_segs=512, H=32, d=128, K=4, seed=601):
    """Conv-coupled exact reuse (conv variant, keys and values from a causal conv over
    C = H (d_k + d_v) raw channels): R requests of 24-96 cached segments (128-1024
    tokens) drawn from a pool whose suffix records were built untimed.  Timed: the
    warmed head keys and values (hypic_conv_kv) and the chains of suffix records with
    the head tokens applied inside the compose (hypic_compose_chain_heads); beside it
    the plain chain of the same records, and the unfused form (a record per head,
    chains of 2m records)."""
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


def cpu_baseline(seg_len=2048, H=32, d=128, nseg_sample=16, seed=301):
    """fp64 oracle on the host: build of nseg_sample of the main workload's 16
    segments, all heads (the first nseg_sample segments' tokens, same seed)."""
    import oracle
    st = synth.gdn_stream([seg_len] * nseg_sample, H, d, d, torch.bfloat16, seed, 0.1, "cpu")
    k, v = st.k.double().numpy(), st.v.double().numpy()
    b, la = st.beta.double().numpy(), st.log_alpha.double().numpy()
    t0 = time.perf_counter()
    oracle.build_segments(oracle.GDN, k, v, la, st.seg_offsets, beta=b)
    dt = time.perf_counter() - t0
    toks = seg_len * nseg_sample
    return {"value": toks / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"GDN build of {nseg_sample} x {seg_len}-token segment(s) x {H} heads, d={d}, "
                      f"fp64 token-by-token recurrence ({dt:.1f} s wall on {oracle.num_threads()} threads)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["all", "main", "sd", "compose", "rag", "convexact", "kda"], default="all",
                    help="main: only the headline GDN step; sd / compose / rag / convexact / kda: it plus that leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one untimed 1 GiB device copy (reference kernel for HBM byte counters)")
    args = ap.parse_args()
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
    ms_step, N, kern, flops, b_ms = bench_main(args)
    traffic = TRAFFIC_GDN_BUILD
    secondary = []
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
    cpu = None if args.no_cpu else cpu_baseline()
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
                   "kv_dtype": "bf16", "record_dtype": "fp32", "parallelism": "none (1 GPU)"},
        "roofline": roofline("mfma", flops / (b_ms * 1e-3) / 1e12, PEAK_BF16 / 1e12, "TFLOP/s", traffic),
        "cpu_baseline": cpu,
        "kernels": kern,
        "secondary": secondary,
        "hbm_attainable": attainable,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
