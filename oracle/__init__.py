"""Plain fp64 CPU oracle for the hybrid-attention decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, headers,
tables or helpers with the HIP library; the two meet only through the seeded
input generators in ``synth/``, which hold none of the method's arithmetic.

Every function is the plain definition (or the plain sequential algorithm)
of one step of the decode path, written in NumPy float64, each citing the
source passage it follows.  The pages that describe the system are short
news articles about the TokenSpeed inference engine; they name the pieces
(KV pages, state slots addressed by index, copy-on-write checkpoints, a fused
QK-RMSNorm + partial-RoPE + gate-split prologue, hybrid full-attention / Gated
DeltaNet layers) but print no formula, constant or worked example.  Where the
pages are silent the module docstrings state the reading taken.

Modules
-------
bf16        bfloat16 <-> float64 codec (round to nearest even)
paging      page-table / slot-pool model (integer, bit-exact) and the gather
attention   softmax decode attention over the gathered context, split
            partials and the log-sum-exp merge
prologue    RMSNorm + partial rotary embedding + gate split
gdn         gated delta rule: sequential definition and chunkwise form
speculative draft-verify bookkeeping and rollback by index
radix       what a hybrid prefix-cache lookup returns (brute force)

Parity status: every function here is pinned by the CPU tests under
``tests/test_oracle_*.py`` (closed forms, invariants, brute force, library
special cases).  None is "parity unpinned".
"""

from . import bf16, paging, attention, prologue, gdn, speculative  # noqa: F401
