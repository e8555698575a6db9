"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct fp64 NumPy/Python implementations of what the
paged-attention hot path computes. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import anything here; the
product path (``paged_kv_cache_indirect_amd``) never does, and this package
imports nothing from it.

Modules
-------
``oracle.attention``      gather K/V through the block table, concatenate,
                          exact softmax attention (decode and causal chunked
                          prefill), log-sum-exp partial states and their merge.
``oracle.scatter``        the KV append scatter (slot_mapping write).
``oracle.block_manager``  a pure-Python model of the host block manager
                          (free list, per-sequence tables, refcounts).

Parity status: every function here is pinned by ``tests/test_oracle*.py``
against something other than itself (library SDPA in fp64, brute-force loops,
closed forms, invariances, worked counts printed on the pages). There is no
page-printed numeric attention output, so the attention value itself rests on
the textbook definition plus those pins.
"""
