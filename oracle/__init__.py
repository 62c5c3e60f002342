"""CPU oracle for one round of CodePredictor speculative decoding.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library; its only common input is the ``synth``
generator, which holds none of the method's arithmetic.

The oracle is a plain, slow, obviously correct restatement of the method:

  * ``philox``        Philox4x32-10 counter-based uniforms (Salmon, Moraes,
                      Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3",
                      SC'11), used for every random draw of a frame.
  * ``distributions`` temperature/top-k softmax, inverse-CDF sampling, the
                      min(1, p/q) acceptance test, the norm(max(0, p-q))
                      residual, the greedy argmax-equality verifier.
  * ``decoder``       the CodePredictor decoder: pre-norm RMSNorm, RoPE, GQA
                      causal attention, SwiGLU FFN, one embedding table and one
                      lm_head per RVQ depth.
  * ``spec``          the per-frame loop: prefill, then rounds of draft /
                      verify / accept / commit-and-truncate; the autoregressive
                      loop is the same loop with an empty draft.

Precision: the decoder and the head logits are computed in float64 from the
same (bf16-rounded where the workload is bf16) weights the GPU reads; the
logits are rounded to float32 and every discrete decision (top-k set, argmax,
sampling walk, acceptance ratio, residual) is taken in float32, the precision
in which the GPU path takes it.

Pins (tests that tie each function to something other than itself) are listed
in the module docstrings; every function here is pinned.
"""
