"""GPU checks of the decode kernel's longest-first workgroup order.

When every sequence of a batch fits one partition and the launch has at
least four workgroups per CU (the dispatcher then hands them out in turns),
workgroup r takes the r-th longest sequence, ties to the lower index (up to
256 sequences every workgroup ranks the batch; larger batches are sorted
once per call, by a one-workgroup sort kernel, into the call's workspace).  Each output row must still be its own sequence's
attention ("KV Cache 和 vLLM" §1.2-1.3: out = softmax(q K^T / sqrt(d)) V over
the sequence's cached tokens).  Batches in that regime - ragged with ties
and an empty sequence, from 40 to 3000 sequences, one already longest first,
and fp8 and int8 + int4 caches - are checked against the fp64 oracle; the
order changes no output bit (a call without a workspace runs in index order);
the fused step, which writes the step's K/V row through the same sequence
index, is checked bit for bit against append-then-decode.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_160_amd as pkv
import workloads as wl
from oracle import scenario
from paged_kv_cache_160_amd.workload_runner import GpuWorkload
from tests._parity import TOL, check_cache_rows, max_err, out_to_f64, say

pytestmark = pytest.mark.gpu


def _lens(kind: str, n: int, seed: int, lmax: int):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, lmax, n)
    lens[3] = 0                                  # an empty sequence
    lens[5] = lens[9] = lens[n - 1] = lens[7]    # ties
    if kind == "sorted":
        lens = np.sort(lens)[::-1]
    return [int(x) for x in lens]


CASES = [  # (kind, num_seqs, hq, hkv, head_dim, source dtype, longest context + 1, cache dtype)
    ("ragged", 40, 32, 32, 64, "bf16", 400, None),
    ("ragged", 100, 32, 16, 64, "f16", 400, None),
    ("ragged", 200, 8, 8, 64, "bf16", 400, None),
    ("sorted", 64, 16, 16, 128, "bf16", 400, None),
    ("ragged", 48, 32, 32, 128, "f32", 400, "fp8_e4m3"),
    ("ragged", 48, 32, 32, 64, "f32", 400, "int8_int4"),
    ("ragged", 600, 8, 2, 64, "bf16", 200, None),
    ("ragged", 3000, 4, 1, 64, "bf16", 80, None),
    # the largest batch the order kernel sorts, and one more (index order)
    ("ragged", 8192, 4, 1, 64, "bf16", 40, None),
    ("ragged", 8193, 4, 1, 64, "bf16", 40, None),
]


def _workload(case, seed=23):
    kind, n, hq, hkv, d, dtype, lmax, cache = case
    return wl.custom_workload(n, hq, hkv, d, _lens(kind, n, seed, lmax), dtype=dtype, cache_dtype=cache,
                              q_dtype="bf16" if cache else None, seed=seed,
                              extra_blocks=4 * n + 8)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[3]}-{c[7] or c[5]}" for c in CASES])
def test_longest_first_rows_match_oracle(case):
    w = _workload(case)
    ops = wl.setup_ops(w)
    seqs = list(range(w.num_seqs))
    say(f"[order] {case}")
    g = GpuWorkload(w).run(ops)
    st = scenario.OracleState(w, build_pool=False).run(ops)
    tables = g.cache.block_tables(seqs)
    ot, ol = st.tables(seqs)
    assert np.array_equal(tables[1].cpu().numpy(), ol)
    # the regime: one partition per sequence, >= 4 workgroups per CU
    _, n_parts = pkv.decode_partition_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, int(tables[2]),
                                           g.cache.cache_code)
    assert n_parts == 1 and w.num_seqs * w.num_kv_heads >= 1024
    out = out_to_f64(g.cache.decode(g.queries(0), 0, tables=tables))
    torch.cuda.synchronize()
    exp = scenario.expected_decode_rows(w, wl.queries(w, 0), seqs, ol)
    err = max_err(out, exp)
    say(f"[order] {case[0]} {case[1]}: max abs err {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL[w.cache_dtype]
    for b in seqs:
        if ol[b] == 0:
            assert np.all(out[b] == 0.0)         # an empty sequence


def test_longest_first_fused_step_equals_append_then_decode():
    w = _workload(CASES[0])
    w.decode_appends = 2
    ops = wl.setup_ops(w)
    seqs = list(range(w.num_seqs))
    say("[order] fused step in longest-first order")
    sep = GpuWorkload(w).run(ops)
    fus = GpuWorkload(w).run(ops)
    for step in range(2):
        sep.append_one_each(seqs)
        out_a = sep.cache.decode(sep.queries(step), 0, seq_ids=seqs)
        out_b = fus.decode_step(seqs, step)
        torch.cuda.synchronize()
        assert torch.equal(out_a.cpu(), out_b.cpu()), f"step {step}"
    ta, la = sep.cache.alloc.block_tables(seqs)
    tb, lb = fus.cache.alloc.block_tables(seqs)
    assert torch.equal(ta, tb) and torch.equal(la, lb)
    for b in seqs:
        check_cache_rows(w, fus.cache, 0, b, tb[b].numpy(), int(lb[b]))


@pytest.mark.parametrize("case", [CASES[6], CASES[7], CASES[8]], ids=["600x2", "3000x1", "8192x1"])
def test_order_changes_no_output_bit(case):
    # the same call with the sorted order (workspace given) and in index
    # order (no workspace): every workgroup computes its row the same way
    w = _workload(case)
    g = GpuWorkload(w).run(wl.setup_ops(w))
    c = g.cache
    seqs = list(range(w.num_seqs))
    bt, lens, max_len = c.block_tables(seqs)
    q = g.queries(0)
    B, hq, hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    need = pkv.workspace_size(B, hq, hkv, D, max_len, 0, c.cache_code)
    assert need > pkv.WS_COUNTER_BYTES          # the launch takes the order
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    lib = pkv._lib.lib()
    sp = torch.cuda.current_stream().cuda_stream
    outs = []
    for wp, wb in ((ws.data_ptr(), need), (None, 0)):
        out = torch.empty_like(q)
        rc = lib.paged_attention_decode_bs(out.data_ptr(), q.data_ptr(), c.k[0].data_ptr(), c.v[0].data_ptr(),
                                           None, None, bt.data_ptr(), lens.data_ptr(), B, hq, hkv, D,
                                           w.num_blocks, w.block_size, w.max_blocks_per_seq, max_len,
                                           1.0 / math.sqrt(D), pkv.dtype_code(q.dtype), c.cache_code, 0, wp, wb, sp)
        assert rc == 0
        outs.append(out.cpu())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    # the order the kernel wrote is the longest-first permutation
    order = ws[pkv.WS_COUNTER_BYTES:pkv.WS_COUNTER_BYTES + 4 * B].view(torch.int32).cpu().numpy()
    ln = lens.cpu().numpy()
    expect = sorted(range(B), key=lambda b: (-int(ln[b]), b))
    assert order.tolist() == expect
