"""Shared helpers for the GPU parity tests: build an engine from seeded inputs,
hand host copies of the same inputs to the oracle, compare results."""
import numpy as np
import torch

import synth
from oracle import model as OM
from oracle.numerics import bf16_bits_to_f64
from speculative_decoding_verify_spec_amd.engine import VerifyEngine

NEAR_TIE = 1e-4      # decisions this close to their boundary may differ
# nucleus cuts this close (in renormalised mass) to top_p may differ: the GPU
# sums fp32 exp() values in fp64, each within a few 1e-7 of the oracle's fp64
# exp (the logit / temperature division in fp32 included)
ADJUST_BAND = 1e-5
LOGIT_RTOL = 2e-2    # per row: max|z_gpu - z_oracle| / max|z_oracle|


def dev():
    return torch.device("cuda:0")


def build_engine(shape, max_batch, max_ctx, max_rows, ctx_len, seed_w=synth.SEED_WEIGHTS,
                 seed_kv=synth.SEED_KV, poison=True):
    names, w = synth.make_weights(shape, seed=seed_w, device=dev())
    cache = synth.make_kv_cache(shape, max_batch, max_ctx, ctx_len, seed=seed_kv, device=dev(),
                                poison_tail=poison)
    eng = VerifyEngine(shape, w, cache, max_batch, max_ctx, max_rows)
    return eng, names, w, cache


def oracle_weights(names, w):
    return OM.Weights(names, [synth.to_numpy_raw(t) for t in w])


def oracle_cache(cache, shape, max_batch, max_ctx):
    k, v = synth.kv_views(cache, shape, max_batch, max_ctx)
    return synth.to_numpy_raw(k).copy(), synth.to_numpy_raw(v).copy()


def logits_rel_err(z_gpu, z_orc):
    z_gpu = np.asarray(z_gpu, np.float64).reshape(-1, z_orc.shape[-1])
    z_orc = np.asarray(z_orc, np.float64).reshape(-1, z_orc.shape[-1])
    num = np.abs(z_gpu - z_orc).max(axis=1)
    den = np.abs(z_orc).max(axis=1)
    return num / den


def compare_decisions(gpu_out, gpu_n, orc, label=""):
    """Token ids must be equal unless the oracle's decision trace has a margin
    below NEAR_TIE.  Returns the number of counted near-tie differences."""
    near = 0
    for b in range(len(gpu_n)):
        same = (int(gpu_n[b]) == int(orc["n_accepted"][b])) and \
            np.array_equal(np.asarray(gpu_out[b]), orc["out_tokens"][b])
        if same:
            continue
        m = min(orc["margins"][b]) if orc["margins"][b] else np.inf
        am = min(orc.get("adjust_margins", [[]] * len(gpu_n))[b], default=np.inf)
        assert m < NEAR_TIE or am < ADJUST_BAND, (
            f"{label} seq {b}: gpu n={gpu_n[b]} out={list(gpu_out[b])} vs oracle "
            f"n={orc['n_accepted'][b]} out={list(orc['out_tokens'][b])}, min margin {m}, nucleus margin {am}")
        near += 1
    return near


def bf16_close(a_bits, b_bits, max_frac=2e-2, noise=1e-4):
    """bf16 rounding of the GPU's K/V vs the oracle's: the two sides round
    values that differ by the forward's numerical noise (about 1e-5 of the
    values' RMS after a layer with d=4096, growing with depth), so a few
    tenths of a percent of elements straddle a rounding boundary.  Bound: at
    most one bf16 ulp (2^-7 |x|) plus `noise` times the RMS, on under
    `max_frac` of the elements.  A wrong row would be off by about the RMS."""
    diff = np.asarray(a_bits) != np.asarray(b_bits)
    assert diff.mean() < max_frac, diff.mean()
    fa, fb = bf16_bits_to_f64(a_bits), bf16_bits_to_f64(b_bits)
    rms = np.sqrt(np.mean(fb * fb))
    tol = 2.0 ** -7 * np.maximum(np.abs(fa), np.abs(fb)) + noise * rms
    worst = np.abs(fa - fb) - tol
    assert np.all(worst <= 0), f"bf16 values apart beyond one ulp + {noise} rms: {worst.max()}"
