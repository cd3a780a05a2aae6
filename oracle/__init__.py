"""CPU oracle for the EntropyCache denoising step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what one denoising
step computes, written from the EntropyCache explainer pages (gist.science
paper 2603.18489: the Italian summary, section "Algoritmo di Funzionamento",
and the Arabic technical summary, section 2 "Algorithm workflow" with its
max-entropy equation). Everything is evaluated in float64; for bf16 models the
oracle rounds to bf16 exactly where the device path stores bf16 ("mirror"
mode), so that the two can be compared element by element.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path never calls it, and it
shares no code with the HIP library; the seeded inputs it consumes come from
the separate ``synth`` package.

Modules:
  entropy  -- per-row softmax entropy, argmax and max-probability (the
              decision signal E).
  model    -- the bidirectional transformer forward over a set of rows with a
              per-layer K/V cache (refresh = all rows, skip = partial rows).
  loop     -- the denoising loop: decode, entropy, threshold decision,
              recompute set of masked + k most recently decoded positions.
  drift    -- the KV-drift measure (cosine distance of cached vs recomputed
              K / V rows), the quantity the pages correlate with E.

Parity pins: every function here is pinned by tests in tests/test_oracle_*.py
against closed forms, library routines or brute force; the end-to-end
trajectory has no worked example on the pages and is pinned only through the
invariants of its parts (parity unpinned beyond those).
"""
from . import entropy, model, loop, drift  # noqa: F401
