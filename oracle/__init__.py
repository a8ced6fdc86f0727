"""CPU oracle of the PB-LRU KV residency engine. TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the engine
computes, written from the UlaCache summary (paper-daily.com, "UlaCache:
Unified Logical Addressing for Sparse LLM Serving", sections 2 and 3) and the
readings stated in each function. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The engine in
``serving_pb_lru_amd`` never imports it, and this package imports nothing of
the engine: the two share only the seeded inputs of ``synth``.

Modules:
    pblru      -- the PB-LRU replacement state of one layer group, in full-data
                  mode (pools hold real bytes) or metadata mode (no pools)
    exact_lru  -- the exact LRU the pages compare against (timestamp per slot,
                  full scan for victims), for the differential tests
    invariants -- the structural invariants checked after every step
    replay     -- runs a synthetic trace through an oracle group

Pinning (what fixes this oracle other than itself): the hand-worked example
under tests/golden, the special case "ring longer than the trace" where PB-LRU
must equal exact LRU bit for bit, the special case of a one-bucket ring, the
special case "pool holds everything" where the gather is a plain fancy index,
the closed-form row contents, the invariants, and the pages' claim that the
hit rate stays within 0.1 percentage point of exact LRU. Some points the pages
leave open (first-occurrence order, miss/victim pairing, the placement of
appended entries, the initial residents, the capacity error): no page passage
decides them, so they are choices stated in this package, which the HIP engine
implements independently; the checks above (the worked examples field by field,
the exact-LRU equivalences, the error-path tests) still pin the functions that
carry them.
"""
