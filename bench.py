#!/usr/bin/env python3
"""Benchmark of the speculative verify step on one MI355X.

Workload (default): Llama-3-8B-shaped decoder with random-init bf16 weights,
B = 1, synthetic bf16 KV context of 2048 tokens, chain verify at gamma = 3
(T = 4 rows), noisy-target drafts with logit noise sigma = 1.0, temperature 1.

One timed step = spec_verify_step (T = gamma + 1 rows, all weights streamed
once) + spec_accept (accept / residual resample / bonus) + the commit of
kv_len, on device-resident inputs.  R pre-drafted rounds from the same cache
state are cycled so acceptance varies; the commit writes to a separate length
buffer so every step sees the same context.

Printed JSON line:
  value         accepted tokens / s = sum_b (n_b + 1) over the timed steps / time
  c_verify      T_verify(gamma+1) / T_decode(1): the same spec_verify_step at
                T = gamma+1 and at T = 1 (same B, context), whole-step times
  roofline      the gate/up GEMM (the largest weight stream): algorithmic bytes
                per launch / mean launch time, from one pair of HIP events
                around its 32 layers' launches run back to back at B*T rows;
                traffic = the HBM bytes the profiler's counters saw per launch,
                read from the committed counter summary while the GEMM source
                still matches the hash recorded there, else null
  cpu_baseline  the CPU oracle timed on this host on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PKG_CSRC = os.path.join(ROOT, "speculative_decoding_verify_spec_amd", "csrc")
# the GEMM kernels' sources: whole files, or (file, first line, end line) for
# the GEMM section of the shared parameter header
GEMM_SOURCES = ("gemm.hip", "common.h", ("launch.h", "-- GEMM\n", "-- attention\n"))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_llama8b_m4_hbm_traffic.txt")


def gemm_sources_sha256():
    """Hash of the GEMM kernel's sources with comments and blank space
    removed (an edited explanation does not change the kernel); the committed
    counter summary is valid only while it matches."""
    import hashlib
    import re

    h = hashlib.sha256()
    for src in GEMM_SOURCES:
        f, first, end = (src, None, None) if isinstance(src, str) else src
        with open(os.path.join(PKG_CSRC, f)) as fh:
            text = fh.read()
        if first is not None:
            # the lines from the section banner ending in `first` up to the next
            # banner ending in `end`
            a = text.index(first)
            text = text[a:text.index(end, a)]
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def committed_traffic(rows):
    """HBM bytes per gate/up launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the same counter's
    reading on a copy of known size), or None when it was taken at another
    row count or on other kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("gemm_sources_sha256") != gemm_sources_sha256() or int(kv.get("rows", -1)) != rows:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128,
                    help="timed steps; by default they cover every pre-drafted round once")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--ctx", type=int, default=2048)
    ap.add_argument("--gamma", type=int, default=3)
    ap.add_argument("--sigma", type=float, default=1.0)
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--top-k", type=int, default=0, help="top-k adjustment of the target (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="top-p adjustment of the target (1: off); the synthetic drafts stay unadjusted")
    ap.add_argument("--rounds", type=int, default=0,
                    help="distinct pre-drafted rounds cycled (0: enough for 128 sequence-rounds, at least 2)")
    ap.add_argument("--sweep", action="store_true",
                    help="B=1 table over gamma in {0,1,3,5,7} x sigma in {0.5,1,2}: c_v, T_verify, tok/s")
    ap.add_argument("--ragged-lens", type=str, default="",
                    help="comma-separated per-sequence verify lengths (one per sequence of --batch): also time "
                         "the compact ragged forward against the fixed-width one")
    ap.add_argument("--ragged-tier", type=int, default=8, help="packed rows are padded to a multiple of this")
    ap.add_argument("--paged", type=int, default=0,
                    help="1: a paged KV cache (64-slot pages, a random block table) instead of the dense one; "
                         "the CPU baseline is then skipped")
    ap.add_argument("--tree", type=str, default="",
                    help="comma-separated branching per depth (e.g. 4,4,2,2): measure token-tree verify instead "
                         "of the chain")
    ap.add_argument("--recurrent", type=int, default=0,
                    help="N > 0: time verify + commit of a recurrent (gated delta-rule) layer for N sequences "
                         "instead of the 8B model (32 heads of 128, 4-tap conv, T = gamma + 1)")
    ap.add_argument("--toy", action="store_true",
                    help="the 2-layer fp32 toy decoder instead of the 8B shape: a real 32-token prefill, then live "
                         "gamma=4 rounds (draft, verify, accept, commit) at temperature 1 and greedy, every round "
                         "replayed end to end by the oracle (--rounds, default 100)")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="1: time the oracle on this host")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the streaming-read ceiling at the 8B GEMMs' weight sizes")
    ap.add_argument("--gemm-route", type=int, default=0,
                    help="GEMM kernel override for A/B timing (spec_gemm_route): 0 automatic, 1 32-row tiles, "
                         "2 large tiles, 3 large tiles in the 4-wave form")
    ap.add_argument("--profile-steps", type=int, default=10)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run an fp32 copy of this many MiB three times first (HBM counter calibration)")
    ap.add_argument("--cpu-seqs", type=int, default=0,
                    help="the oracle leg runs only the first N sequences of the batch (0: all); its tok/s is that "
                         "subset's own, and the decision checks cover the same sequences")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle rounds are repeated until this much CPU time is spent (at most 3)")
    return ap.parse_args()


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the verify step of this build runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import speculative_decoding_verify_spec_amd as S
    from speculative_decoding_verify_spec_amd.engine import VerifyEngine

    S.lib()  # fail loudly when the HIP library is missing
    if a.gemm_route:
        S.spec_gemm_route(a.gemm_route)
    dev = torch.device("cuda:0")
    if a.recurrent:
        return run_recurrent(a, dev)
    if a.toy:
        return run_toy(a, dev)
    if a.read_ceiling:
        sizes = {"o": 4096 * 4096 * 2, "qkv": 6144 * 4096 * 2, "down": 4096 * 14336 * 2,
                 "gate_up": 28672 * 4096 * 2, "lm_head": 128256 * 4096 * 2}
        res = read_ceiling(S, dev, sizes)
        print(json.dumps({"metric": "streaming-read ceiling (launch to end, back to back)", "unit": "us",
                          "sizes": res}), flush=True)
        return
    sh = synth.LLAMA8B
    if a.rounds <= 0:
        a.rounds = max(2, -(-128 // a.batch))
    if a.sweep:
        a.gamma = max(SWEEP_GAMMAS)
    B, ctx, gamma, T = a.batch, a.ctx, a.gamma, a.gamma + 1
    if a.tree:
        branching = [int(x) for x in a.tree.split(",")]
        T = int(synth.random_tree(branching, 1).shape[1])
    max_ctx = ((ctx + T + 63) // 64) * 64
    log(f"workload: {sh.n_layers}L d={sh.d_model} V={sh.vocab} B={B} ctx={ctx} gamma={gamma}")

    t0 = time.time()
    names, w = synth.make_weights(sh, device=dev)
    if a.paged:
        # a pool of 64-slot pages; each sequence's pages in a seeded random order
        pps = max_ctx // 64
        kv_pages = B * pps + 8
        cache = synth.make_kv_pool(sh, kv_pages, device=dev)
        eng = VerifyEngine(sh, w, cache, B, max_ctx, max(T, 1), kv_pages=kv_pages)
        eng.set_block_table(synth.random_block_table(B, pps, kv_pages).to(dev))
        a.cpu_baseline = 0
    else:
        cache = synth.make_kv_cache(sh, B, max_ctx, ctx, device=dev, poison_tail=False)
        eng = VerifyEngine(sh, w, cache, B, max_ctx, max(T, 1))
    torch.cuda.synchronize()
    log(f"weights + cache ready in {time.time() - t0:.1f}s")

    if a.calibrate_copy_mib > 0:
        # a plain elementwise pass of known size: per dispatch it reads and
        # writes exactly n * 4 bytes, which scales the profiler's HBM counters
        # (a negation, so that its kernel is easy to tell from the others)
        n = a.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {n * 4} bytes read and written")
        del src, dst

    kv_len = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    kv_out = torch.empty_like(kv_len)
    pending = synth.make_tokens(B, 1, sh.vocab, seed=synth.SEED_PROMPT, device=dev)
    if a.tree:
        return run_tree(a, sh, eng, names, w, cache, kv_len, pending, dev)
    if a.sweep:
        return run_sweep(a, sh, eng, kv_len, pending, dev)

    rounds = draft_rounds(eng, sh, B, gamma, a.sigma, a.temperature, a.rounds, kv_len, pending, dev)
    log(f"{a.rounds} draft rounds ready")

    logits = torch.empty((B, T, sh.vocab), device=dev)
    out = torch.empty((B, T), dtype=torch.int32, device=dev)
    nacc_hist = torch.zeros((a.steps + a.warmup, B), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_step(k):
        tokens, qt = rounds[k % len(rounds)]
        eng.step(tokens, kv_len, logits)
        eng.accept(logits, qt if gamma else None, tokens, out, nacc_hist[k], kv_len, kv_out,
                   temperature=a.temperature, seed=synth.SEED_ACCEPT, round_=k, top_k=a.top_k, top_p=a.top_p)

    for k in range(a.warmup):
        one_step(k)
    torch.cuda.synchronize()
    # one event between consecutive steps: the per-step distribution
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i, k in enumerate(range(a.warmup, a.warmup + a.steps)):
        one_step(k)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0].elapsed_time(evs[-1])
    step_ms = step_percentiles(evs)
    n_timed = nacc_hist[a.warmup:].cpu().numpy()
    tokens_out = int((n_timed + 1).sum())
    value = tokens_out / wall
    ms_per_step = wall * 1000.0 / a.steps
    acc_stats = acceptance_stats(n_timed, gamma, a.sigma, a.temperature)
    assert eng.device_errors() == 0
    log(f"timed {a.steps} steps: {ms_per_step:.3f} ms/step (events {gpu_ms / a.steps:.3f}), "
        f"{tokens_out} tokens, {value:.1f} tok/s")

    # ---- c = T_verify(gamma+1) / T_decode(1), whole-step times
    def time_forward(Tn, iters):
        tok = rounds[0][0][:, :Tn].contiguous()
        lg = torch.empty((B, Tn, sh.vocab), device=dev)
        for _ in range(3):
            eng.step(tok, kv_len, lg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            eng.step(tok, kv_len, lg)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    iters = max(10, a.steps // 2)
    t_verify = time_forward(T, iters)
    t_decode = time_forward(1, iters)
    c_v = t_verify / t_decode
    log(f"T_verify({T}) {t_verify:.3f} ms, T_decode(1) {t_decode:.3f} ms, c = {c_v:.3f}")

    # ---- ragged verify: compact forward of the packed lengths (padded to the
    # execution tier) against the fixed-width forward at T = max length
    ragged = None
    if a.ragged_lens:
        lens = [int(x) for x in a.ragged_lens.split(",")]
        assert len(lens) == B and all(1 <= n <= T for n in lens), "one length in [1, gamma+1] per sequence"
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        rows = int(-(-int(cu[-1]) // a.ragged_tier) * a.ragged_tier)
        cu_d = torch.from_numpy(cu).to(dev)
        tok_r = torch.cat([rounds[0][0][b, :lens[b]] for b in range(B)]
                          + [rounds[0][0][0, :1].expand(rows - int(cu[-1]))]).contiguous()
        lg_r = torch.empty((rows, sh.vocab), device=dev)
        for _ in range(3):
            eng.step_ragged(cu_d, max(lens), tok_r, kv_len, lg_r)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            eng.step_ragged(cu_d, max(lens), tok_r, kv_len, lg_r)
        e1.record(stream)
        torch.cuda.synchronize()
        t_compact = e0.elapsed_time(e1) / iters
        ragged = {"lens": lens, "total_verify_tokens": int(cu[-1]), "graph_num_tokens": rows,
                  "t_compact_ms": round(t_compact, 4), "t_fixed_width_ms": round(t_verify, 4),
                  "fixed_width_rows": B * T}
        log(f"ragged lens {lens}: compact {t_compact:.3f} ms ({rows} rows) vs fixed width {t_verify:.3f} ms "
            f"({B * T} rows)")

    # ---- roofline of the dominant kernel (the gate/up GEMM, the largest weight
    # stream): its launches for all 32 layers back to back at the verify's
    # B*T rows, bracketed by one pair of HIP events on the launch stream
    iters_gu = 4
    gu_ms, gu_bytes = eng.profile_gemm("gemm_gate_up", B * T, iters_gu)
    n_gu = iters_gu * sh.n_layers
    gu_avg_s = gu_ms * 1e-3 / n_gu
    gu_bytes_launch = gu_bytes / n_gu
    roofline = {"bound": "hbm", "kernel": "gemm_gate_up (skinny-M weight stream, fused RMSNorm + SiLU*up)",
                "achieved": round(gu_bytes_launch / gu_avg_s / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gu_bytes_launch / gu_avg_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": committed_traffic(B * T), "algo_bytes_per_launch": gu_bytes_launch,
                "avg_launch_us": round(gu_avg_s * 1e6, 3), "launches_timed": n_gu}
    log(f"gate/up GEMM: {roofline['avg_launch_us']} us/launch, {roofline['achieved']} GB/s")
    # the same bytes as one plain streaming read: what a kernel of this size
    # reaches at best, launch, ramp and tail included
    rc = read_ceiling(S, dev, {"gate_up": int(gu_bytes_launch) // 16 * 16})["gate_up"]
    roofline["read_ceiling"] = {**rc, "frac_of_ceiling": round(rc["us"] / roofline["avg_launch_us"], 4)}
    log(f"read ceiling at {rc['bytes']} B: {rc['us']} us ({rc['GBps']} GB/s)")

    # ---- per-kernel-class event timing (a separate profiled pass)
    kernels = {}
    if a.profile_steps > 0:
        # the pass reuses the accept-count rows of the timed steps
        kernels, agg = profile_pass(S, eng, lambda k: one_step(k % (a.steps + a.warmup)), a.profile_steps)
        roofline.update(agg)

    result = {
        "metric": "verify cost ratio c=T_verify/T_decode; accepted tok/s; HBM GB/s vs peak",
        "value": round(value, 2), "unit": "accepted tok/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "step_ms": step_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (bf16 weights, fp32 activations/accum)",
        "data": "synthetic (random-init weights, random bf16 KV context, noisy-target drafts)",
        "config": {"workload": f"llama3-8b-shape chain verify B={B} ctx={ctx} gamma={gamma} "
                               f"sigma={a.sigma} T={a.temperature}"
                               + (f" top_k={a.top_k}" if a.top_k else "")
                               + (f" top_p={a.top_p}" if a.top_p < 1.0 else "")
                               + (" paged-kv(64)" if a.paged else ""),
                   "B": B, "ctx": ctx, "gamma": gamma, "sigma": a.sigma, "temperature": a.temperature,
                   "top_k": a.top_k, "top_p": a.top_p, "parallelism": "single GPU"},
        "c_verify": round(c_v, 4), "t_verify_ms": round(t_verify, 4), "t_decode_ms": round(t_decode, 4),
        "rounds": {"distinct": a.rounds, "sequences_per_round": B, "timed_sequence_rounds": int(n_timed.size)},
        **acc_stats,
        "kernels": kernels, "roofline": roofline,
    }
    if ragged is not None:
        result["ragged"] = ragged

    if a.cpu_baseline:
        # the GPU's decisions the oracle leg compares with: every timed step's
        # logits and accept output (shared-logits tier), and round 0 accepted
        # with each uniform round the oracle's own forward is used for
        # the oracle's sequences: the first nb of the batch (rows are
        # independent; the uniforms are indexed by sequence)
        nb = min(B, a.cpu_seqs) if a.cpu_seqs > 0 else B
        nk = min(a.steps, 128)
        shared = []
        for k in range(a.warmup, a.warmup + nk):
            one_step(k)
            tokens, qt = rounds[k % len(rounds)]
            shared.append((k, tokens[:nb].cpu().numpy(), qt[:nb].double().cpu().numpy() if gamma else None,
                           logits[:nb].double().cpu().numpy(), out[:nb].cpu().numpy(),
                           nacc_hist[k][:nb].cpu().numpy()))
        e2e = []
        for j in range(3):
            tokens, qt = rounds[0]
            eng.step(tokens, kv_len, logits)
            eng.accept(logits, qt if gamma else None, tokens, out, nacc_hist[0], kv_len, kv_out,
                       temperature=a.temperature, seed=synth.SEED_ACCEPT, round_=j, top_k=a.top_k, top_p=a.top_p)
            e2e.append((out[:nb].cpu().numpy(), nacc_hist[0][:nb].cpu().numpy()))
        result["cpu_baseline"], result["near_ties"] = cpu_baseline(sh, names, w, cache, B, max_ctx, ctx, rounds[0], a,
                                                                   kv_len, shared, e2e, nb)
    print(json.dumps(result), flush=True)


SWEEP_GAMMAS = (0, 1, 3, 5, 7)
SWEEP_SIGMAS = (0.5, 1.0, 2.0)


def draft_rounds(eng, sh, B, gamma, sigma, temperature, R, kv_len, pending, dev):
    """R rounds pre-drafted from the same state: gamma sequential T=1 decodes
    give the target logits z_i of each drafted prefix; the noisy-target draft
    is q_i = softmax(z_i + eps), eps ~ N(0, sigma^2), x_i ~ q_i (argmax of the
    noisy logits at temperature 0).  Untimed: the draft is synthetic."""
    import torch

    import synth

    rounds = []
    z1 = torch.empty((B, 1, sh.vocab), device=dev)
    for r in range(R):
        toks = [pending[:, 0]]
        qs = []
        for i in range(gamma):
            tok = toks[-1][:, None].contiguous().to(torch.int32)
            eng.step(tok, kv_len + i, z1)
            q, zn = synth.noisy_draft_dist(z1[:, 0], sigma, synth.SEED_NOISE * 1000 + r * 16 + i,
                                           temperature if temperature > 0 else 1.0)
            if temperature > 0:
                x = synth.sample_from(q, synth.SEED_DRAFT * 1000 + r * 16 + i)[:, 0]
            else:
                x = zn.argmax(-1).to(torch.int32)
            toks.append(x)
            qs.append(q)
        tokens = torch.stack(toks, 1).to(torch.int32).contiguous()
        qt = torch.stack(qs, 1).contiguous() if gamma and temperature > 0 else \
            torch.empty((B, 0, sh.vocab), device=dev)
        rounds.append((tokens, qt))
    torch.cuda.synchronize()
    return rounds


def acceptance_stats(n, gamma, sigma, temperature):
    """Per-position acceptance alpha = tests passed / tests reached (a round
    that accepted n < gamma drafts reached n + 1 tests, one that accepted all
    reached gamma), its closed form for the noisy-target draft at temperature
    1, 2 Phi(-sigma/2) (flat target logits), and tokens per round against
    eq. (1) of CS349E Lecture 6 section 8.1 at the measured alpha."""
    import numpy as np

    n = np.asarray(n).ravel()
    out = {"mean_accepted": round(float(n.mean()), 4), "tokens_per_round": round(float((n + 1).mean()), 4)}
    if gamma == 0:
        return out
    passed = int(n.sum())
    reached = int(np.minimum(n + 1, gamma).sum())
    alpha = passed / reached if reached else 0.0
    out["alpha_per_position"] = round(alpha, 4)
    out["alpha_se"] = round(math.sqrt(max(alpha * (1 - alpha), 0.0) / max(reached, 1)), 4)
    if temperature > 0:
        out["alpha_closed_form"] = round(math.erfc(sigma / 2.0 / math.sqrt(2.0)), 4)  # 2 Phi(-sigma/2)
    out["tokens_per_round_eq1"] = round((1 - alpha ** (gamma + 1)) / (1 - alpha) if alpha < 1 else gamma + 1.0, 4)
    out["tokens_per_round_se"] = round(float((n + 1).std(ddof=1) / math.sqrt(n.size)) if n.size > 1 else 0.0, 4)
    return out


def run_sweep(a, sh, eng, kv_len, pending, dev):
    """The B=1 table over draft length and draft quality: for each gamma, the
    whole-step T_verify(gamma+1) and c_v = T_verify / T_decode(1); for each
    (gamma, sigma), accepted tok/s over timed verify + accept steps cycling
    pre-drafted rounds (the DeepSeek-V4 analysis page's step cost against the
    verify window; the verify-cost page's decode steps per verify)."""
    import torch

    import synth

    B, V = a.batch, sh.vocab
    stream = torch.cuda.current_stream(dev)

    def time_forward(tok, iters=20):
        lg = torch.empty((B, tok.shape[1], V), device=dev)
        for _ in range(3):
            eng.step(tok, kv_len, lg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            eng.step(tok, kv_len, lg)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    R = max(16, a.rounds // 2)
    table = []
    kv_out = torch.empty_like(kv_len)
    t_decode = None
    for gamma in SWEEP_GAMMAS:
        T = gamma + 1
        logits = torch.empty((B, T, V), device=dev)
        out = torch.empty((B, T), dtype=torch.int32, device=dev)
        for sigma in SWEEP_SIGMAS:
            rounds = draft_rounds(eng, sh, B, gamma, sigma, a.temperature, R, kv_len, pending, dev)
            if t_decode is None:
                t_decode = time_forward(rounds[0][0][:, :1].contiguous())
            t_verify = time_forward(rounds[0][0])
            nacc = torch.zeros((2 * R, B), dtype=torch.int32, device=dev)

            def one_step(k):
                tokens, qt = rounds[k % R]
                eng.step(tokens, kv_len, logits)
                eng.accept(logits, qt if gamma and a.temperature > 0 else None, tokens, out, nacc[k], kv_len,
                           kv_out, temperature=a.temperature, seed=synth.SEED_ACCEPT, round_=k)

            for k in range(4):
                one_step(k)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(R, 2 * R):
                one_step(k)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            n = nacc[R:].cpu().numpy()
            row = {"gamma": gamma, "sigma": sigma, "t_verify_ms": round(t_verify, 4),
                   "t_decode_ms": round(t_decode, 4), "c_v": round(t_verify / t_decode, 4),
                   "ms_per_step": round(wall * 1000.0 / R, 4),
                   "tok_s": round(float((n + 1).sum()) / wall, 2),
                   **acceptance_stats(n, gamma, sigma, a.temperature)}
            table.append(row)
            log(f"gamma {gamma} sigma {sigma}: c_v {row['c_v']}, {row['tok_s']} tok/s, "
                f"{row['tokens_per_round']} tokens/round")
    assert eng.device_errors() == 0
    print(json.dumps({
        "metric": "verify cost ratio c=T_verify/T_decode; accepted tok/s (sweep)", "unit": "accepted tok/s",
        "n_gpus": 1, "higher_is_better": True, "vs_baseline": None,
        "dtype": "f32 (bf16 weights, fp32 activations/accum)",
        "data": "synthetic (random-init weights, random bf16 KV context, noisy-target drafts)",
        "config": {"workload": f"llama3-8b-shape chain verify B={B} ctx={a.ctx} gamma x sigma sweep "
                               f"T={a.temperature}", "B": B, "ctx": a.ctx, "rounds_per_point": R,
                   "parallelism": "single GPU"},
        "sweep": table}), flush=True)


def run_tree(a, sh, eng, names, w, cache, kv_len, pending, dev):
    """Token-tree verify (CS349E Lecture 6, section 10.3): B sequences, each a
    full tree with the given branching per depth.  Drafting (untimed): level
    by level, the verify forward gives every node's target logits, the draft
    distribution of a node is q = softmax(z + noise) and its children are drawn
    from q without replacement.  Timed: verify + tree accept (+ path commit to
    a separate length buffer, so the context stays fixed)."""
    import numpy as np
    import torch

    import synth

    branching = [int(x) for x in a.tree.split(",")]
    B, V = a.batch, sh.vocab
    parent = synth.random_tree(branching, B).to(dev)
    T = int(parent.shape[1])
    ch = synth.tree_children(parent[0].cpu().tolist())
    depth = [0] * T
    for v in range(1, T):
        depth[v] = depth[int(parent[0, v])] + 1
    log(f"tree {branching}: {T} nodes per sequence, {B * T} rows")
    logits = torch.empty((B, T, V), device=dev)
    rounds = []
    g = torch.Generator(device="cpu")
    for r in range(a.rounds):
        tokens = torch.zeros((B, T), dtype=torch.int32, device=dev)
        tokens[:, 0] = pending[:, 0]
        q = None
        for lvl in range(len(branching)):
            eng.step(tokens, kv_len, logits, tree_parent=parent)
            q, zn = synth.noisy_draft_dist(logits, a.sigma, synth.SEED_NOISE * 1000 + r * 16 + lvl,
                                           a.temperature if a.temperature > 0 else 1.0)
            g.manual_seed(synth.SEED_DRAFT * 1000 + r * 16 + lvl)
            qc = q.double().cpu()
            zc = zn.cpu()
            tk = tokens.cpu()
            for b in range(B):
                for v in range(T):
                    if depth[v] == lvl and ch[v]:
                        if a.temperature > 0:  # children drawn from q without replacement
                            picks = torch.multinomial(qc[b, v], len(ch[v]), replacement=False, generator=g)
                        else:  # greedy: the draft's top-k
                            picks = torch.topk(zc[b, v], len(ch[v])).indices
                        for c, x in zip(ch[v], picks.tolist()):
                            tk[b, c] = x
            tokens = tk.to(dev)
        rounds.append((tokens.contiguous(), q.contiguous()))
    torch.cuda.synchronize()
    log(f"{a.rounds} tree rounds drafted")
    out = torch.empty((B, T), dtype=torch.int32, device=dev)
    nacc_hist = torch.zeros((a.steps + a.warmup, B), dtype=torch.int32, device=dev)
    kv_out = torch.empty_like(kv_len)
    stream = torch.cuda.current_stream(dev)

    def one_step(k):
        tokens, q = rounds[k % len(rounds)]
        eng.step(tokens, kv_len, logits, tree_parent=parent)
        eng.accept(logits, q if a.temperature > 0 else None, tokens, out, nacc_hist[k], kv_len, kv_out,
                   tree_parent=parent, temperature=a.temperature, seed=synth.SEED_ACCEPT, round_=k)

    for k in range(a.warmup):
        one_step(k)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i, k in enumerate(range(a.warmup, a.warmup + a.steps)):
        one_step(k)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = step_percentiles(evs)
    n_timed = nacc_hist[a.warmup:].cpu().numpy()
    tokens_out = int((n_timed + 1).sum())
    ms_per_step = wall * 1000.0 / a.steps

    def time_forward(tok, par, iters=10):
        lg = torch.empty((B, tok.shape[1], V), device=dev)
        for _ in range(3):
            eng.step(tok, kv_len, lg, tree_parent=par)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            eng.step(tok, kv_len, lg, tree_parent=par)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    t_verify = time_forward(rounds[0][0], parent)
    t_decode = time_forward(rounds[0][0][:, :1].contiguous(), None)
    kernels = {}
    if a.profile_steps > 0:
        import speculative_decoding_verify_spec_amd as S
        kernels, _ = profile_pass(S, eng, lambda k: one_step(k % (a.steps + a.warmup)), a.profile_steps)
    assert eng.device_errors() == 0
    result = {
        "metric": "verify cost ratio c=T_verify/T_decode; accepted tok/s; HBM GB/s vs peak",
        "value": round(tokens_out / wall, 2), "unit": "accepted tok/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4), "step_ms": step_ms, "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 (bf16 weights, fp32 activations/accum)",
        "data": "synthetic (random-init weights, random bf16 KV context, noisy-target tree drafts)",
        "config": {"workload": f"llama3-8b-shape tree verify B={B} ctx={a.ctx} tree={branching} ({T} nodes) "
                               f"sigma={a.sigma} T={a.temperature}",
                   "B": B, "ctx": a.ctx, "tree": branching, "nodes": T, "sigma": a.sigma,
                   "temperature": a.temperature, "parallelism": "single GPU"},
        "c_verify": round(t_verify / t_decode, 4), "t_verify_ms": round(t_verify, 4),
        "t_decode_ms": round(t_decode, 4), "mean_accepted": round(float(n_timed.mean()), 4),
        "tokens_per_round": round(float((n_timed + 1).mean()), 4), "kernels": kernels,
    }
    log(f"tree: {ms_per_step:.3f} ms/step, {result['value']} tok/s, T_verify {t_verify:.3f} ms, "
        f"T_decode {t_decode:.3f} ms")
    print(json.dumps(result), flush=True)


def run_recurrent(a, dev):
    """Verify on a recurrent layer (Kimi-K3 tuning page, "Verification on a
    recurrent layer is not a cache write"): N sequences, a window of
    T = gamma + 1 positions, 32 heads of width 128, a 4-tap conv.  One step =
    spec_recurrent_verify over the window + spec_recurrent_commit of the
    survivor after a synthetic accept count per sequence, with the pool
    resident in HBM.  Both ways of recovering the survivor are timed: keeping
    the T candidate states (snapshots, the pages' engines) and replaying the
    committed positions at commit time, and the fused call that commits the
    previous window and verifies the next in one kernel; `value` is the fused
    step, the others are reported beside it.  A step commits to a copy of the
    pool, so every step starts from the same state."""
    import numpy as np
    import torch

    import synth
    import speculative_decoding_verify_spec_amd as S

    rs = synth.RECURRENT_8B
    B, T = a.recurrent, a.gamma + 1
    H, D, W = rs.n_heads, rs.head_dim, rs.conv_width
    log(f"recurrent workload: B={B} T={T} H={H} D={D} W={W}")
    inp = synth.make_recurrent_inputs(rs, B, T, B)
    d = {k: v.to(dev).contiguous() for k, v in inp.items()}
    dims = S.spec_recurrent_dims(H, D, W, B)
    out = torch.empty((B, T, H, D), device=dev)
    snaps = torch.empty((B, T, H, D, D), device=dev)
    cs, st = d["conv_state"].clone(), d["state"].clone()
    g = torch.Generator().manual_seed(synth.SEED_ACCEPT)
    naccs = [torch.randint(0, T, (B,), generator=g, dtype=torch.int32).to(dev) for _ in range(8)]
    stream = torch.cuda.current_stream(dev)

    def verify(keep):
        S.spec_recurrent_verify(dims, B, T, d["x"], d["gate"], d["beta"], d["conv_w"], None, d["conv_state"],
                                d["state"], out, snaps if keep else None, stream)

    def commit(keep, k):
        S.spec_recurrent_commit(dims, B, T, d["x"], d["gate"], d["beta"], d["conv_w"], None, naccs[k % 8],
                                snaps if keep else None, cs, st, stream)

    def timed(fn, iters):
        for k in range(3):
            fn(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(iters):
            fn(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def step(keep):
        def f(k):
            verify(keep)
            commit(keep, k)
        return f

    def fused(k):
        # one round in steady state: the previous window's commit and this
        # window's verify in one call (the same synthetic window stands for both)
        S.spec_recurrent_commit_verify(dims, B, T, d["x"], d["gate"], d["beta"], naccs[k % 8], T, d["x"], d["gate"],
                                       d["beta"], d["conv_w"], None, cs, st, out, stream)

    for _ in range(a.warmup):
        step(True)(0)
        step(False)(0)
    torch.cuda.synchronize()
    ms_snap = timed(step(True), a.steps)
    ms_replay = timed(step(False), a.steps)
    ms_fused = timed(fused, a.steps)
    # per-kernel averages, launches back to back between one pair of events
    iters = max(a.steps, 20)
    us = {"verify_snapshots": timed(lambda k: verify(True), iters) * 1e3,
          "verify": timed(lambda k: verify(False), iters) * 1e3,
          "commit_scatter": timed(lambda k: commit(True, k), iters) * 1e3,
          "commit_replay": timed(lambda k: commit(False, k), iters) * 1e3,
          "commit_verify": ms_fused * 1e3}
    # algorithmic bytes (fp32): the state D x D per (sequence, head), the
    # window's raw channels, gates and betas, the outputs
    st_b = B * H * D * D * 4
    win_b = B * T * (3 * H * D + H * D + H) * 4
    conv_b = B * (W - 1) * 3 * H * D * 4
    out_b = B * T * H * D * 4
    nbar = float(torch.stack(naccs).float().mean()) + 1.0  # committed positions per sequence
    algo = {"verify_snapshots": st_b + T * st_b + win_b + conv_b + out_b,
            "verify": st_b + win_b + conv_b + out_b,
            "commit_scatter": 2 * st_b + 2 * conv_b,
            "commit_replay": 2 * st_b + win_b * nbar / T + 2 * conv_b,
            "commit_verify": 2 * st_b + win_b * nbar / T + win_b + 3 * conv_b + out_b}
    kern = {k: {"avg_us": round(us[k], 3), "algo_bytes": int(algo[k]),
                "GBps": round(algo[k] / (us[k] * 1e-6) / 1e9, 1)} for k in us}
    for k, v in kern.items():
        log(f"{k}: {v['avg_us']} us, {v['GBps']} GB/s")
    # the step that value reports: one fused call per round (the previous
    # window's replay commit, then this window's verify; the same results as
    # the separate calls, bit for bit), a single kernel
    dom = "commit_verify"
    roofline = {"bound": "hbm", "kernel": "rec_commit_verify_kernel (previous survivor replayed and stored, "
                                          "new window verified)",
                "achieved": kern[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kern[dom]["GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                "algo_bytes_per_launch": algo[dom], "avg_launch_us": kern[dom]["avg_us"]}
    value = B * T / (ms_fused * 1e-3)
    result = {
        "metric": "recurrent-state verify: window positions verified per second (verify + survivor commit)",
        "value": round(value, 1), "unit": "window positions/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_fused, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (random window inputs and states)",
        "config": {"workload": f"recurrent gated delta-rule verify B={B} T={T} H={H} D={D} conv={W}",
                   "B": B, "T": T, "heads": H, "head_dim": D, "conv_width": W, "parallelism": "single GPU"},
        "commit": "fused (commit of the previous window + verify)",
        "ms_per_step_replay": round(ms_replay, 4),
        "value_replay": round(B * T / (ms_replay * 1e-3), 1),
        "ms_per_step_snapshots": round(ms_snap, 4),
        "value_snapshots": round(B * T / (ms_snap * 1e-3), 1),
        "kernels": kern, "roofline": roofline,
    }
    if a.cpu_baseline:
        from oracle import recurrent as OR
        n = min(B, 4)
        h = {k: v[:n].double().numpy() if k not in ("conv_w",) else v.double().numpy() for k, v in inp.items()}
        nacc = naccs[0][:n].cpu().numpy()
        t0, reps = time.perf_counter(), 0
        while reps == 0 or time.perf_counter() - t0 < a.cpu_seconds:
            o, sn = OR.verify(h["x"], h["gate"], h["beta"], h["conv_w"], h["conv_state"], h["state"])
            OR.commit(h["x"], nacc, h["conv_state"], h["state"], sn)
            reps += 1
        dt = time.perf_counter() - t0
        threads = None
        try:
            from threadpoolctl import threadpool_info
            threads = max((q.get("num_threads") or 0) for q in threadpool_info()) or None
        except Exception:
            pass
        result["cpu_baseline"] = {"value": round(n * T * reps / dt, 2), "unit": "window positions/s",
                                  "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
                                  "sample": f"{reps} windows of {n} sequences (the first {n} of the workload), "
                                            f"verify + snapshot commit; {dt:.1f} s"}
    log(f"recurrent: {ms_fused:.4f} ms/step (fused), {ms_replay:.4f} (replay), {ms_snap:.4f} (snapshots)")
    print(json.dumps(result), flush=True)


TOY_PROMPT, TOY_GAMMA = 32, 4


def run_toy(a, dev):
    """The toy decoder (2 layers, d=256, 4 heads of 64, FFN 1024, vocab 4096,
    fp32 weights), B=1: the step prefills a 32-token prompt itself, then R
    live rounds at gamma=4 each draft with gamma T=1 decodes of the target
    (noisy-target draft, sigma), verify the window, accept and commit
    kv_len, the emitted token becoming the next pending one (CS349E
    Lecture 6, section 6.2).  Temperature 1 and greedy are both run.

    Timing: the recorded rounds are replayed in order (verify + accept, the
    round's kv_len restored; the draft is synthetic and untimed), which also
    checks that a replay reproduces the live round bit for bit.  The oracle
    replays every round end to end from its own prefill and its own commits,
    with the round's drafted tokens, q and Philox uniforms, until the first
    round whose results differ (counted as a near tie or a mismatch)."""
    import numpy as np
    import torch

    import synth
    from speculative_decoding_verify_spec_amd.engine import VerifyEngine

    sh = synth.TOY
    gamma, T = TOY_GAMMA, TOY_GAMMA + 1
    R = a.rounds if a.rounds > 0 else 100
    max_ctx = ((TOY_PROMPT + R * T + T + 63) // 64) * 64
    log(f"workload: toy {sh.n_layers}L d={sh.d_model} V={sh.vocab} fp32, prompt {TOY_PROMPT}, gamma={gamma}, "
        f"{R} rounds")
    names, w = synth.make_weights(sh, device=dev)
    cache = synth.make_kv_cache(sh, 1, max_ctx, 0, device=dev, poison_tail=False)
    eng = VerifyEngine(sh, w, cache, 1, max_ctx, TOY_PROMPT)
    prompt = synth.make_tokens(1, TOY_PROMPT, sh.vocab, seed=synth.SEED_PROMPT, device=dev)

    def live(temp):
        return toy_live(eng, sh, prompt, R, temp, a.sigma, dev)

    def replay(temp, recs, first):
        lg = torch.empty((1, T, sh.vocab), device=dev)
        out = torch.empty((1, T), dtype=torch.int32, device=dev)
        nacc = torch.empty((R,), dtype=torch.int32, device=dev)
        kv_out = torch.empty((1,), dtype=torch.int32, device=dev)
        kvs = [torch.tensor([rc["kv"]], dtype=torch.int32, device=dev) for rc in recs]
        same = True
        for k in range(a.warmup):  # untimed; the replay restores each round's kv_len
            rc = recs[k % R]
            eng.step(rc["tokens"], kvs[k % R], lg)
            eng.accept(lg, rc["q"], rc["tokens"], out, nacc[k % R:k % R + 1], kvs[k % R], kv_out,
                       temperature=temp, seed=synth.SEED_ACCEPT, round_=k % R)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for r, rc in enumerate(recs):
            eng.step(rc["tokens"], kvs[r], lg)
            eng.accept(lg, rc["q"], rc["tokens"], out, nacc[r:r + 1], kvs[r], kv_out, temperature=temp,
                       seed=synth.SEED_ACCEPT, round_=r)
            if first:
                same = same and bool(torch.equal(lg, rc["logits"])) and bool(torch.equal(out, rc["out"]))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        n = nacc.cpu().numpy()
        return wall, n, same

    modes = {}
    for temp in (1.0, 0.0):
        _, recs = live(temp)
        n_live = np.array([rc["n"] for rc in recs])
        wall, n_rep, same = replay(temp, recs, True)
        assert (n_rep == n_live).all() and same, "replayed rounds differ from the live ones"
        wall2, _, _ = replay(temp, recs, False)  # timed without the comparisons
        toks = int((n_live + 1).sum())
        modes[temp] = {"recs": recs, "value": toks / wall2, "ms_per_round": wall2 * 1e3 / R,
                       "stats": acceptance_stats(n_live, gamma, a.sigma, temp)}
        log(f"toy T={temp}: {R} rounds, {toks} tokens, {wall2 * 1e3 / R:.3f} ms per verify + accept, "
            f"{toks / wall2:.1f} tok/s; replay identical to the live rounds")
    assert eng.device_errors() == 0

    # ---- c = T_verify(gamma+1) / T_decode(1) at the prompt's end
    stream = torch.cuda.current_stream(dev)

    def time_forward(Tn, iters=200):
        tok = modes[1.0]["recs"][0]["tokens"][:, :Tn].contiguous()
        lg = torch.empty((1, Tn, sh.vocab), device=dev)
        kvt = torch.tensor([TOY_PROMPT], dtype=torch.int32, device=dev)
        for _ in range(5):
            eng.step(tok, kvt, lg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            eng.step(tok, kvt, lg)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    t_verify, t_decode = time_forward(T), time_forward(1)
    log(f"toy T_verify({T}) {t_verify * 1e3:.1f} us, T_decode(1) {t_decode * 1e3:.1f} us, "
        f"c = {t_verify / t_decode:.3f}")

    m1 = modes[1.0]
    result = {
        "metric": "verify cost ratio c=T_verify/T_decode; accepted tok/s; HBM GB/s vs peak",
        "value": round(m1["value"], 2), "unit": "accepted tok/s", "n_gpus": 1, "steps": R, "warmup": a.warmup,
        "ms_per_step": round(m1["ms_per_round"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (random-init fp32 weights, uniform random prompt, noisy-target drafts)",
        "config": {"workload": f"toy decoder 2L d=256 fp32 chain verify B=1 prompt={TOY_PROMPT} gamma={gamma} "
                               f"sigma={a.sigma} T=1.0 (greedy beside it)",
                   "B": 1, "prompt": TOY_PROMPT, "gamma": gamma, "sigma": a.sigma, "rounds": R,
                   "parallelism": "single GPU"},
        "c_verify": round(t_verify / t_decode, 4), "t_verify_ms": round(t_verify, 5),
        "t_decode_ms": round(t_decode, 5), **m1["stats"],
        "greedy": {"value": round(modes[0.0]["value"], 2), "ms_per_step": round(modes[0.0]["ms_per_round"], 4),
                   **modes[0.0]["stats"]},
        "bound": "latency (the whole model, 12.6 MB of fp32 weights, sits in the caches)",
    }
    if a.cpu_baseline:
        result["cpu_baseline"], result["near_ties"] = toy_oracle(sh, names, w, prompt, modes)
    print(json.dumps(result), flush=True)


def toy_live(eng, sh, prompt, R, temp, sigma, dev):
    """Prefill the prompt with the step itself, then R live rounds of the toy
    workload (see run_toy); returns the last pending token and the records."""
    import torch

    import synth

    gamma, T = TOY_GAMMA, TOY_GAMMA + 1
    z1 = torch.empty((1, 1, sh.vocab), device=dev)
    zp = torch.empty((1, TOY_PROMPT, sh.vocab), device=dev)
    eng.step(prompt, torch.zeros(1, dtype=torch.int32, device=dev), zp)
    pending = int(zp[0, -1].argmax())
    kv = TOY_PROMPT
    recs = []
    for r in range(R):
        kvt = torch.tensor([kv], dtype=torch.int32, device=dev)
        toks, qs = [pending], []
        for i in range(gamma):
            eng.step(torch.tensor([[toks[-1]]], dtype=torch.int32, device=dev), kvt + i, z1)
            q, zn = synth.noisy_draft_dist(z1[:, 0], sigma, synth.SEED_NOISE * 1000 + r * 16 + i,
                                           temp if temp > 0 else 1.0)
            x = int(synth.sample_from(q, synth.SEED_DRAFT * 1000 + r * 16 + i)[0, 0]) if temp > 0 \
                else int(zn[0].argmax())
            toks.append(x)
            qs.append(q)
        tokens = torch.tensor([toks], dtype=torch.int32, device=dev)
        qt = torch.stack(qs, 1).contiguous() if temp > 0 else None
        lg = torch.empty((1, T, sh.vocab), device=dev)
        out = torch.empty((1, T), dtype=torch.int32, device=dev)
        nacc = torch.empty((1,), dtype=torch.int32, device=dev)
        kv_out = torch.empty((1,), dtype=torch.int32, device=dev)
        eng.step(tokens, kvt, lg)
        eng.accept(lg, qt, tokens, out, nacc, kvt, kv_out, temperature=temp, seed=synth.SEED_ACCEPT, round_=r)
        n = int(nacc[0])
        assert int(kv_out[0]) == kv + n + 1
        recs.append({"kv": kv, "tokens": tokens, "q": qt, "logits": lg, "out": out, "n": n})
        pending = int(out[0, n])
        kv += n + 1
    torch.cuda.synchronize()
    return pending, recs


def toy_oracle(sh, names, w, prompt, modes):
    """The oracle's own prefill and rounds, end to end, against the GPU's live
    rounds (same drafted tokens, q and uniforms; the oracle commits its own
    accepted prefix).  Stops at the first round whose results differ."""
    import numpy as np

    import synth
    from oracle import accept as OA
    from oracle import model as OM
    from oracle import philox

    W = OM.Weights(names, [synth.to_numpy_raw(t) for t in w])
    L, H, D = sh.n_layers, sh.n_kv_heads, sh.head_dim
    dt, toks, rounds_timed = 0.0, 0, 0
    report = {}
    for temp, m in modes.items():
        recs = m["recs"]
        max_ctx = TOY_PROMPT + len(recs) * (TOY_GAMMA + 1) + TOY_GAMMA + 1
        kc = np.zeros((L, 1, H, max_ctx, D), dtype=np.uint16)
        vc = np.zeros((L, 1, H, D, max_ctx), dtype=np.uint16)
        pt = prompt.cpu().numpy()
        z, kn, vn = OM.forward(sh, W, pt, np.array([0]), kc, vc)
        OM.write_suffix(kc, vc, kn, vn, np.array([0]))
        pending = int(np.argmax(z[0, -1]))
        kv = np.array([TOY_PROMPT])
        counts, compared, first_diff, max_err = [0, 0, 0], 0, None, 0.0
        for r, rc in enumerate(recs):
            tokens = rc["tokens"].cpu().numpy()
            if int(tokens[0, 0]) != pending or int(kv[0]) != rc["kv"]:
                first_diff = first_diff if first_diff is not None else r
                break
            t0 = time.perf_counter()
            z, kn, vn = OM.forward(sh, W, tokens, kv, kc, vc)
            OM.write_suffix(kc, vc, kn, vn, kv)
            q = rc["q"].double().cpu().numpy() if rc["q"] is not None else None
            res = OA.accept(z, q, tokens, temp, philox.Uniforms(synth.SEED_ACCEPT, r))
            dt += time.perf_counter() - t0
            rounds_timed += 1
            toks += int(res["n_accepted"][0]) + 1
            zg = rc["logits"].double().cpu().numpy()
            max_err = max(max_err, float(np.max(np.abs(zg - z)) / np.max(np.abs(z))))
            g_out, g_n = rc["out"].cpu().numpy(), np.array([rc["n"]])
            c = count_decisions(g_out, g_n, res, draw_band=1e-4)
            for i, x in enumerate(c):
                counts[i] += x
            compared += 1
            if c[1] or c[2]:
                first_diff = r
                break
            n = int(res["n_accepted"][0])
            pending = int(res["out_tokens"][0][n])
            kv = OM.commit_chain(kv, res["n_accepted"])
        report["temperature_1" if temp > 0 else "greedy"] = {
            "rounds_compared": compared, "rounds": len(recs), "decisions": counts[0],
            "near_tie_differences": counts[1], "mismatches": counts[2], "first_differing_round": first_diff,
            "max_logits_rel_err": float(f"{max_err:.3g}"), "draw_band": 1e-4, "band": 1e-4}
        log(f"toy oracle T={temp}: {compared}/{len(recs)} rounds compared end to end, decisions {counts}, "
            f"logits rel err {max_err:.2e}")
    cores = len(os.sched_getaffinity(0))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    base = {"value": round(toks / dt, 2), "unit": "accepted tok/s", "cores": threads or cores, "kind": "oracle",
            "sample": f"{rounds_timed} verify rounds of the toy (forward over 5 rows + accept, temperature 1 and "
                      f"greedy), end to end; {dt:.2f} s", "host_cores_visible": cores,
            "threads_note": "cores = the BLAS threads the oracle ran on (threadpoolctl), else the visible cores"}
    return base, {"end_to_end": report}


def read_ceiling(S, dev, sizes, iters=None):
    """Best launch-to-end time of a plain streaming read of each size (bytes)
    over a few launch shapes, through the library's measurement hook."""
    import torch

    span = 3 << 30
    raw = torch.empty(span + 4096, dtype=torch.uint8, device=dev)
    pad = (-raw.data_ptr()) % 4096
    buf = raw[pad:pad + span]
    out = {}
    for name, nbytes in sizes.items():
        best = None
        for grid in (256, 512, 1024, 2048):
            for unroll in (4, 8):
                it = iters or (20 if nbytes > (256 << 20) else 100)
                us = S.spec_profile_stream_read(buf, nbytes, it, grid, unroll)
                if best is None or us < best[0]:
                    best = (us, grid, unroll)
        us, grid, unroll = best
        out[name] = {"bytes": nbytes, "us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1), "grid": grid,
                     "unroll": unroll}
    del raw, buf
    torch.cuda.empty_cache()
    return out


def step_percentiles(evs):
    """Median, P10 and P90 of the step times between consecutive HIP events
    recorded on the launch stream (ms)."""
    import numpy as np

    d = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)])
    return {"median": round(float(np.median(d)), 4), "p10": round(float(np.percentile(d, 10)), 4),
            "p90": round(float(np.percentile(d, 90)), 4)}


def profile_pass(S, eng, one_step, steps):
    """Per-kernel-class HIP-event timing over `steps` full steps.  Every launch
    is bracketed by its own events, so these averages include the dispatch
    latency in front of each kernel; the aggregate GEMM bandwidth is reported
    beside the roofline figure, which comes from back-to-back launches."""
    import torch

    S.spec_profile_enable(eng.handle, True)
    for k in range(steps):
        one_step(k)
    torch.cuda.synchronize()
    stats = S.spec_profile_read(eng.handle, reset=True)
    S.spec_profile_enable(eng.handle, False)
    kernels = {}
    for name, st in stats.items():
        if st["launches"]:
            avg_ms = st["total_ms"] / st["launches"]
            gbs = st["algo_bytes"] / (st["total_ms"] * 1e-3) / 1e9 if st["total_ms"] > 0 else 0.0
            kernels[name] = {"launches_per_step": st["launches"] / steps,
                             "avg_us": round(avg_ms * 1e3, 3), "algo_GBps": round(gbs, 1)}
    gemm_names = [k for k in stats if k.startswith("gemm_")]
    g_bytes = sum(stats[k]["algo_bytes"] for k in gemm_names)
    g_ms = sum(stats[k]["total_ms"] for k in gemm_names)
    roofline = {"all_gemms_GBps": round(g_bytes / (g_ms * 1e-3) / 1e9, 1),
                "all_gemms_frac": round(g_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return kernels, roofline


def _first_difference(g_out, g_n, o_out, o_n):
    m = min(g_n, o_n)
    for j in range(m + 1):
        if int(g_out[j]) != int(o_out[j]):
            return j
    return m


def count_decisions(gpu_out, gpu_n, orc, draw_band, band=1e-4):
    """The GPU's accept results against the oracle's (same logits, q, drafts
    and uniforms): decisions taken, sequences that differ only at a near-tie of
    their first differing decision (an accept test with |u - min(1, p/q)| <
    band, an argmax with a top-2 gap under band of max|z|, or a final draw
    whose GPU token sits within draw_band * R of u * R on the oracle's CDF),
    and sequences that differ otherwise (mismatches, expected 0)."""
    decisions = near = mismatch = 0
    for b in range(len(gpu_n)):
        g_n, o_n = int(gpu_n[b]), int(orc["n_accepted"][b])
        g_out, o_out = gpu_out[b], orc["out_tokens"][b]
        decisions += len(orc["margins"][b])
        if g_n == o_n and all(int(g_out[i]) == int(o_out[i]) for i in range(g_n + 1)):
            continue
        j = _first_difference(g_out, g_n, o_out, o_n)
        tr = orc["traces"][b]
        draw_k = len(orc["margins"][b]) - 1 if "draw" in tr else -1
        if "draw" in tr and g_n == o_n and j == o_n:
            t, c = tr["draw"]
            y = int(g_out[j])
            R = float(c[-1])
            ok = 0 <= y < len(c) and c[y] > (c[y - 1] if y else 0.0)
            lo, hi = (float(c[y - 1]) if y else 0.0, float(c[y])) if ok else (0.0, 0.0)
            dist = 0.0 if lo <= t < hi else min(abs(t - lo), abs(t - hi))
            excused = ok and dist <= draw_band * R
        else:
            ms = [m for k, (m, d) in enumerate(zip(orc["margins"][b], tr["depths"])) if d == j and k != draw_k]
            excused = min(ms, default=float("inf")) < band
        am = orc["adjust_margins"][b]
        if j < len(am) and am[j] < 1e-5:
            excused = True
        near += int(excused)
        mismatch += int(not excused)
    return decisions, near, mismatch


def cpu_baseline(sh, names, w, cache, B, max_ctx, ctx, round0, a, kv_len, shared, e2e, nb=None):
    """One verify round (forward over the T rows + accept) of the same workload
    in the CPU oracle, on this host's cores.  The oracle's results also give
    the decision check the benchmark spec asks to report: the GPU's accept on its
    own logits against the oracle's accept on the same logits for the timed
    steps (shared-logits tier), and the GPU's round-0 decisions against the
    oracle's forward + accept of round 0 (end-to-end tier)."""
    import numpy as np

    import synth
    from oracle import accept as OA
    from oracle import model as OM
    from oracle import philox

    log("cpu baseline: copying weights and cache to host")
    nb = B if nb is None else nb
    Wn = OM.Weights(names, [synth.to_numpy_raw(t) for t in w])
    k, v = synth.kv_views(cache, sh, B, max_ctx, seqs=nb)
    kc, vc = synth.to_numpy_raw(k), synth.to_numpy_raw(v)
    del k, v
    tokens, qt = round0
    tok = tokens[:nb].cpu().numpy()
    qn = qt[:nb].double().cpu().numpy() if a.gamma and a.temperature > 0 else None
    cores = len(os.sched_getaffinity(0))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    log(f"cpu baseline: oracle rounds on {cores} cores")
    dt, toks, nrounds = 0.0, 0, 0
    e2e_counts = [0, 0, 0]
    while nrounds < 3 and (nrounds == 0 or dt < a.cpu_seconds):
        t0 = time.perf_counter()
        z, _, _ = OM.forward(sh, Wn, tok, np.full(nb, ctx), kc, vc)
        res = OA.accept(z, qn, tok, a.temperature, philox.Uniforms(synth.SEED_ACCEPT, nrounds),
                        top_k=a.top_k, top_p=a.top_p)
        dt += time.perf_counter() - t0
        toks += int((res["n_accepted"] + 1).sum())
        g_out, g_n = e2e[nrounds]
        for i, x in enumerate(count_decisions(g_out, g_n, res, draw_band=1e-4)):
            e2e_counts[i] += x
        nrounds += 1
    log(f"cpu baseline: {dt:.1f}s for {nrounds} rounds, {toks} tokens")
    sh_counts = [0, 0, 0]
    for kk, tk, qq, zz, g_out, g_n in shared:
        res = OA.accept(zz, qq, tk, a.temperature, philox.Uniforms(synth.SEED_ACCEPT, kk), top_k=a.top_k,
                        top_p=a.top_p)
        for i, x in enumerate(count_decisions(g_out, g_n, res, draw_band=1e-6)):
            sh_counts[i] += x
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    base = {"value": round(toks / dt, 4), "unit": "accepted tok/s", "cores": threads or cores, "cpu_model": cpu_model,
            "kind": "oracle", "sample": f"{nrounds} verify rounds (" + (f"the first {nb} of the B={B} sequences"
                                                                      if nb < B else f"B={B}")
                                        + f", T={a.gamma + 1}, ctx {ctx}, 32 layers, forward + accept) of the "
                                        f"same workload; {dt:.1f} s",
            "round_seconds": round(dt / nrounds, 2), "host_cores_visible": cores,
            "threads_note": "cores = the BLAS threads the oracle ran on (threadpoolctl), else the visible cores"}
    near = {"shared_logits": {"sequence_rounds": len(shared) * nb, "decisions": sh_counts[0],
                              "near_tie_differences": sh_counts[1], "mismatches": sh_counts[2],
                              "draw_band": 1e-6, "band": 1e-4},
            "end_to_end": {"sequence_rounds": nrounds * nb, "decisions": e2e_counts[0],
                           "near_tie_differences": e2e_counts[1], "mismatches": e2e_counts[2],
                           "draw_band": 1e-4, "band": 1e-4}}
    log(f"decisions: shared logits {sh_counts}, end to end {e2e_counts} (decisions, near ties, mismatches)")
    return base, near


if __name__ == "__main__":
    main()
