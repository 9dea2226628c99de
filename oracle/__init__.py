"""CPU oracle for the VeriCache draft/verify attention path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The product
path (``kv_cache_compressed_amd`` and its HIP library) never imports, calls or falls back to
it, and this package imports nothing from the product path except the seeded input
generator in ``kv_cache_compressed_amd.synth`` (which holds no step of the method).

What it computes, each step in plain NumPy, float64 unless stated:

* ``quant``     -- KIVI-style asymmetric min/max quantisation (keys per channel over 32-token
                   groups, values per token over 32-channel groups) in exact float32 IEEE
                   steps, the packed code layout the library documents, and dequantisation.
* ``attention`` -- single-query decode attention over an explicit key set (full KV, KIVI
                   dequantised KV + residual, kept-index KV), the multi-query causal verify
                   (row i *is* decode at position n+i), and the log-sum-exp merge of split
                   partials.
* ``accept``    -- per-row argmax (lowest index on ties) and the greedy accept rule.
* ``loop``      -- a tiny autoregressive model used to pin the accept rule through the
                   pages' guarantee (VeriCache emits exactly the full-KV greedy sequence).

Sources: the pages "VeriCache: making lossy KV compression exact" (a blog walk-through),
"VeriCache: Turning Lossy KV Cache into Lossless LLM Inference" (a knowledge-base summary of
the paper) and "KV-Cache Compression" (a knowledge-base concept page). Every function cites
the page and section it follows; where the pages are silent the reading taken is stated.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force, an independent library routine, or the pages' worked
example. The acceptance *rate* on synthetic data is reported only ("parity unpinned"): the
pages' ~0.8 figure is for trained models on real text.
"""
