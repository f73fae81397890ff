"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (``paged_kv_cache_160_amd``) never does, and this package never
imports the product path: the two share no code.  Inputs come from the
separate ``workloads`` module, which holds only seeded random draws.

Contents (each function cites the passage of the pages it follows):
  fp8_e4m3   OCP E4M3FN codec and the per-row quantisation reading
  cache      slot arithmetic, cache writes (copy and fp8), copy-on-write
  attention  softmax(q K^T / sqrt(d)) V in fp64, paged and contiguous forms,
             partition states and their log-sum-exp merge
  allocator  reference model of the block allocator (refcounts, fork, CoW)
  sizing     KV memory formula and utilisation figures

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (library routines, closed forms, worked values printed on
the pages, brute force, invariants); see tests/test_oracle_*.py.
"""
from . import allocator, attention, cache, fp8_e4m3, sizing  # noqa: F401
