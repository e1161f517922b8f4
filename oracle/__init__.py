"""CPU oracle for the packed 2-bit ternary KV cache and decode attention over it.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
anything in this package: only the tests, the package's smoke check and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators).

It is written for obviousness, not speed: NumPy in float64 wherever the pages
leave the precision open, float32 exactly where the encoding fixes it
(the scale gamma and the division x / (gamma + eps)).

Sources (cited by page title and section):
  * "Show HN: Vantage-V-AI" (newshot.cc), section "core architecture":
    ternary states {-1, 0, +1}, per-tensor dynamic scale gamma = mean(|X|),
    four elements per uint8 (2.0 bits/element), 7.97x smaller than FP16,
    attention sinks (sink_tokens = 4) kept beside a bounded recent window.
  * "Minima-KV" (twodots.gr), sections on the Recent/Anchor/Stale tiers and
    on mixed-format attention: FP8 recent pages, higher-fidelity anchor
    pages, packed stale pages, read directly and merged by one online
    softmax in logical page order.

Readings where the pages are silent are listed in each module's docstring.
Parity status: every function here is pinned by tests under tests/ that do
not re-run the oracle's own formula (hand-worked fixtures in tests/golden,
closed forms, exact-rational brute force, library routines).
"""
