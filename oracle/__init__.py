"""CPU oracle for the speculative verify step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy (fp64) implementations of what the verify
path computes, written from the pages:

  * model.py   -- the target model's forward over B sequences x T verify rows
                  (chain or tree), cached context plus speculative suffix;
  * accept.py  -- Leviathan et al.'s speculative-sampling accept / residual
                  resample / bonus (chain and token tree, sampled and greedy)
                  and the pending-token KV commit;
  * philox.py  -- Philox4x64-10 (Salmon et al., SC'11), the uniforms' source;
  * metrics.py -- the closed forms the pages give (beta, tokens per round,
                  speedup, compute increase, accept-rate metrics);
  * numerics.py -- bf16 decoding and round-to-nearest-even;
  * recurrent.py -- verify on a recurrent (gated delta-rule) layer: the state
                  advanced through the window, its snapshots and the
                  post-verify survivor scatter.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the HIP path and imports nothing from it.

Pins: the forward's layer composition agrees with an independent Llama
decoder implementation (the `transformers` library's, tests/test_oracle_hf_llama.py);
its components with closed forms and library routines, and the whole forward
with causal and prefill/decode consistency (tests/test_oracle_model.py); the
accept rule by exact enumeration of chains and small trees with planted wrong
variants as negative controls (tests/test_oracle_pins.py).

Parity unpinned: the absolute logit values of the random-init 8B-shaped model
have no external reference beyond those checks.  The sibling order of a token
tree has no printed example; enumeration pins only losslessness.
"""
from . import philox, numerics, model, accept, metrics, recurrent  # noqa: F401
