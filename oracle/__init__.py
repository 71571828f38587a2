"""CPU oracle of the Qwen3-TTS 12 Hz per-frame generation step.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
reference that the HIP path is checked against. Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and shares no code with it.

It follows the pages' description of the method step by step, in numpy, in
float32 by default (the precision the pages' own parity work uses: PyTorch
fp32 golden references and CPU FP32 strict-parity runs), with float64
available for the pins:

  model.py     RMSNorm, rope, GQA attention, the Qwen3-style decoder layer,
               KV-cached and full-recompute forward passes
  sampling.py  talker/predictor logits processors, warpers and the
               exponential-race single sample
  philox.py    Philox4x64-10 counter-based generator (noise for the race)
  loop.py      prompt prefill, the per-frame loop (talker step, 2-token
               predictor prefill + 14 steps, embedding-sum feedback), stop
               rules and counters
  frontend.py  token-id frontend: text embedding, ResizeMLP, dual-track
               prompt assembly

Pinned by tests/test_oracle_*.py (closed forms, invariants, library
routines, brute force, golden values under tests/golden/). Parity with the
real Qwen3-TTS checkpoints is unpinned: no weights or golden codes exist here.
"""
from .loop import generate, prefill_row, OracleNonFinite  # noqa: F401
from . import model, sampling, philox, frontend  # noqa: F401
