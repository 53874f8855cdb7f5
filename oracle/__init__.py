"""CPU oracle for the chunked-prefill mixed step.  TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The product path (the HIP library and its Python
binding) never touches it, and this package imports nothing from the product path.

Parts, each a plain and slow restatement of what the pages define:

* ``builder``   -- the decode-first, FCFS, token-budget batch builder and its block pool, with
                   the optional caps and priority policies.
* ``rope``      -- the rotary table and its fp32 evaluation; bf16 round-to-nearest-even.
* ``attention`` -- non-chunked full-prefill causal attention in fp64 for any set of rows, and the
                   expected contents of the paged KV cache.
* ``linear``    -- the linear layers around attention (x . w^T in fp64) and the bound a float32
                   sum rounded to bfloat16 stays within.
* ``sim``       -- a step-by-step simulation over the reference builder: time to first token and
                   time between tokens, in steps.

Pinned by the ``-m "not gpu"`` tests against the pages' printed examples, closed forms,
invariants and brute force.  One convention has no pin in the pages: the rotary variant
(rotate-half, base 10000, fp32 table from fp64) -- "parity unpinned" for the choice of variant,
though its arithmetic is pinned against an operation-by-operation float32 emulation.
"""
