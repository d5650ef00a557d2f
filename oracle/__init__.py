"""CPU oracle for the LoLA chunkwise attention step (one layer).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or link anything under ``oracle/``; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code with the HIP path.

Sources cited in this package (the pages are the authority on the method):

* **LoLA notes** -- "LoLA: Low-Rank Linear Attention With Sparse Caching |
  中文精读笔记" (close-reading notes on arXiv:2505.23666v3, cc.laoqi.cc).
  Sections are cited by the notes' own numbering, e.g. "LoLA notes §2.4,
  Eqs. (11)-(13)".
* **LoLA summary** -- "Technical Summary: LoLA: Low-Rank Linear Attention with
  Sparse Caching" (gist.science), sections "The Self-Recall Error (SRE)
  Mechanism" and "Inference Strategy".

Modules:

* :mod:`oracle.lola`   -- chunk-vectorised float64 form (every size).
* :mod:`oracle.brute`  -- scalar-loop form over an explicit token history
  (tiny shapes only); independent bookkeeping (position sets, not arrays).
* :mod:`oracle.token_mode` -- the notes' per-token recurrence (§2.4), used to
  pin the C = 1 state trajectory.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, special-case reductions to textbook attention, invariants,
brute force).  The values of general outputs on random inputs have no printed
worked example on the pages; they are pinned only through those checks.
"""

from .lola import (  # noqa: F401
    LolaState,
    phi,
    sre,
    select_keep,
    prefill,
    decode_step,
    new_state,
    state_elements,
)
