"""Host-side checks of bench.py's bookkeeping (no GPU): the HBM-traffic
summary it reports is keyed to the GEMM sources, and the key can be computed
and the committed summary parsed."""
import re

import bench


def test_gemm_source_key_is_computable():
    # every source, and the GEMM section of the shared parameter header, exists
    assert re.fullmatch(r"[0-9a-f]{64}", bench.gemm_sources_sha256())


def test_traffic_summary_parses_and_matches_row_count():
    t = bench.committed_traffic(4)
    # None only when the committed summary was taken on other GEMM sources
    assert t is None or t > 2.3e8
    assert bench.committed_traffic(5) is None  # taken at 4 rows only


def _oracle_rounds(sh, names, w, prompt, R, temp, gamma):
    """Live rounds produced by the oracle itself, in the record format of the
    toy workload (drafts from the oracle's own decodes, noisy-target q)."""
    import numpy as np
    import torch

    import synth
    from oracle import accept as OA
    from oracle import model as OM
    from oracle import philox

    W = OM.Weights(names, [synth.to_numpy_raw(t) for t in w])
    L, H, D = sh.n_layers, sh.n_kv_heads, sh.head_dim
    n_ctx = bench.TOY_PROMPT + R * (gamma + 1) + gamma + 1
    kc = np.zeros((L, 1, H, n_ctx, D), dtype=np.uint16)
    vc = np.zeros((L, 1, H, D, n_ctx), dtype=np.uint16)
    z, kn, vn = OM.forward(sh, W, prompt.numpy(), np.array([0]), kc, vc)
    OM.write_suffix(kc, vc, kn, vn, np.array([0]))
    pending, kv, recs = int(np.argmax(z[0, -1])), bench.TOY_PROMPT, []
    for r in range(R):
        kd, vd = kc.copy(), vc.copy()
        toks, qs = [pending], []
        for i in range(gamma):
            zi, kn1, vn1 = OM.forward(sh, W, np.array([[toks[-1]]]), np.array([kv + i]), kd, vd)
            OM.write_suffix(kd, vd, kn1, vn1, np.array([kv + i]))
            q, zn = synth.noisy_draft_dist(torch.from_numpy(zi[:, 0]).float(), 1.0, 1000 * r + i,
                                           temp if temp > 0 else 1.0)
            toks.append(int(synth.sample_from(q, 2000 * r + i)[0, 0]) if temp > 0 else int(zn[0].argmax()))
            qs.append(q)
        tokens = np.array([toks], dtype=np.int32)
        z, kn, vn = OM.forward(sh, W, tokens, np.array([kv]), kc, vc)
        OM.write_suffix(kc, vc, kn, vn, np.array([kv]))
        qt = torch.stack(qs, 1) if temp > 0 else None
        res = OA.accept(z, qt.double().numpy() if qt is not None else None, tokens, temp,
                        philox.Uniforms(synth.SEED_ACCEPT, r))
        n = int(res["n_accepted"][0])
        recs.append({"kv": kv, "tokens": torch.from_numpy(tokens), "q": qt, "logits": torch.from_numpy(z),
                     "out": torch.from_numpy(np.asarray(res["out_tokens"], dtype=np.int32)), "n": n})
        pending = int(res["out_tokens"][0][n])
        kv += n + 1
    return recs


def test_toy_oracle_replay_agrees_with_itself_and_stops_at_a_planted_difference():
    """The toy workload's end-to-end oracle replay: rounds the oracle produced
    itself compare equal all the way (zero logits error, no differing
    decision); a round whose recorded emitted token is changed is reported as
    the first differing round and the replay stops there."""
    import synth

    sh = synth.TOY
    names, w = synth.make_weights(sh)
    prompt = synth.make_tokens(1, bench.TOY_PROMPT, sh.vocab, seed=synth.SEED_PROMPT)
    R = 3
    modes = {t: {"recs": _oracle_rounds(sh, names, w, prompt, R, t, bench.TOY_GAMMA)} for t in (1.0, 0.0)}
    base, near = bench.toy_oracle(sh, names, w, prompt, modes)
    for key in ("temperature_1", "greedy"):
        rep = near["end_to_end"][key]
        assert rep["rounds_compared"] == R and rep["first_differing_round"] is None, rep
        assert rep["near_tie_differences"] == 0 and rep["mismatches"] == 0
        assert rep["max_logits_rel_err"] == 0.0
    assert base["value"] > 0
    # plant a wrong emitted token in round 1 of the greedy run
    rc = modes[0.0]["recs"][1]
    rc["out"] = rc["out"].clone()
    rc["out"][0, rc["n"]] = (int(rc["out"][0, rc["n"]]) + 1) % sh.vocab
    _, near = bench.toy_oracle(sh, names, w, prompt, modes)
    rep = near["end_to_end"]["greedy"]
    assert rep["first_differing_round"] == 1 and rep["rounds_compared"] == 2
    assert rep["near_tie_differences"] + rep["mismatches"] == 1
