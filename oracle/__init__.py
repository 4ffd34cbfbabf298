"""Float64 CPU oracle for paged-KV decode -- TEST INFRASTRUCTURE ONLY.

This package is the reference the GPU library is checked against. It is a
plain, slow, obviously correct restatement of what the method computes:

* ``oracle.pool``      -- block allocator with prefix sharing, copy-on-write
                          and release, plus slot mapping and block tables.
* ``oracle.attention`` -- cache write into a host pool and attention that
                          walks each sequence's block table token by token.
* ``oracle.geometry``  -- payload and FLOP counts used as closed-form pins.
* ``oracle.native``    -- a plain C float64 attention walk (OpenMP over
                          rows) for sizes the Python walk cannot reach.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything in this package. The
GPU library never uses it, and it shares no code with the library.

Citations name the pages the method comes from:

* [KVNB §n] -- course page "Module 10. KV Caches and Efficient Inference",
  notebook "KV cache and serving: bytes, pages, and ceilings", section n.
* [KVNB demo] -- the same page, "Module 10 project-exercise demo".
* [vLLM abstract] -- the PagedAttention / vLLM abstract on the papers search
  page for "external vector cache".
* [NeuralOps] -- "NeuralOps v1.3.4: Serving Primitives & KV Cache
  Optimization", "Architectural Breakdown", item 1 "Paged KV Cache Engine".

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, library routines or brute
force; none is "parity unpinned".
"""
