"""CPU oracle for TurboQuant KV-cache quantize-on-write and compressed-KV decode attention.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, fp64 numpy
implementation of what the GPU path computes, written from the pages and
sharing no code, header, table or constant generator with the HIP library.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it; the product path never does.

Modules
  lloyd_max  Gaussian Lloyd-Max codebook ("Closing - The Three-Step Summary", Step 2).
  rotation   Walsh-Hadamard rotation with random signs ("Closing - The Three-Step
             Summary", Step 1; "What the Paper Doesn't Tell You", Finding 4).
  codec      norm / rotate / quantize / QJL residual sketch and the packed page
             layout ("Closing - The Three-Step Summary", Steps 1-3; "Where This
             Fits in the Inference Stack", sections on tensor parallelism and
             Blackwell FP4 for table-lookup indices; "Why the KV Cache Exists",
             section on PagedAttention).
  attention  brute-force GQA decode attention over the dequantized cache, and
             the same result computed in the rotated domain ("Why the KV Cache
             Exists", sections "The KV Cache Solution" and "What's in the KV Cache").
  dense      the uncompressed (bf16) paged cache and decode attention over it:
             the comparator's oracle ("Where This Fits in the Inference Stack",
             "What Changes When KV Cache Is 4x Smaller").

Every function is pinned by tests under ``tests/`` that check it against closed
forms, textbook tables, library routines and brute force rather than against
itself. Functions without such a pin say "parity unpinned" in their docstring.
"""
from . import lloyd_max, rotation, codec, attention  # noqa: F401
