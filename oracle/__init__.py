"""Plain CPU oracle for block-causal sink + sliding-window attention over a
bounded KV cache (JoyAI-Video-Edit's chunk-wise attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (``block_causal_kv_amd`` and its HIP library) never does, and this
package never imports the product path: the two share no code.

Everything is written to be checked by eye against the pages:

* ``mask``      - which keys a query of chunk c may see (the visibility rule).
* ``attention`` - naive softmax attention under an explicit boolean mask, fp64.
* ``stream``    - per-chunk attention over [cond | clean chunks 0..c-1 | chunk c].
* ``cache``     - a plain list model of the bounded cache (slots, FIFO eviction).
* ``fp8``       - the OCP e4m3 ("E4M3FN") codec and per-block quantisation.

Sources (page title, section):

* JoyAI-Video-Edit tutorial (agifrontier.github.io), section "From bidirectional
  editing to a chunk-wise causal architecture": bidirectional inside a chunk,
  causal across chunks, a fixed window of recent history chunks, and the first
  chunk resident as a global sink.
* Same page, section "Hardware-software co-deployment", bullet "constant KV
  cache": clean K/V are written to the cache after a chunk is generated; the
  cache is always sink + sliding window, so KV memory and compute stay level.
* neurohive.io review, section "Chunks and fighting drift": the active chunk
  looks at a fixed number of recent chunks plus the very first one; section
  "Architecture", figure caption: the mask shows which token groups (condition
  tokens included) the active chunk can see.
* zhichai.net post, paragraph "first axe": only the last few history chunks
  plus the first chunk are kept, so the work per chunk is constant.

Parity status of every function is listed in the module docstrings; all are
pinned by tests in ``tests/test_oracle_*.py``.
"""
