"""CPU oracle for PagedAttention decode — TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product library never
calls it, and it shares no code with the HIP path: everything here is written
out plainly, in float64, from the pages' description of the method:

* "vLLM in Production — PagedAttention, Continuous Batching, and
  OpenAI-Compatible LLM Serving" (datasops.com), sections "The KV Cache and the
  60–80% Memory Tax" and "PagedAttention — Virtual Memory for the KV Cache";
* "Serving models with vLLM" (allaboutaibydeep.pages.dev), sections
  "How it works: PagedAttention" and "See it in code";
* "What Is vLLM: The Fast Inference Engine for Large Language Models"
  (fp8.co), section "How does PagedAttention work?".

Modules:

``attention``    paged decode attention: gather each sequence's keys and
                 values through its block table, then softmax(q·Kᵀ·scale)·V.
``cache_write``  the cache write of new tokens through a slot mapping.
``allocator``    the block allocator: fixed-size blocks handed out on demand,
                 a per-sequence block table, shared prefix blocks counted by
                 reference.

Every function is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, library routines or brute force; none is marked
"parity unpinned".
"""
