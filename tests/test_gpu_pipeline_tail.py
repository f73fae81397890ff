"""GPU parity of the decode pipeline's last tiles for 16-bit and fp32 caches.

A wave takes every fourth 16-token tile of its partition and ends with a
straight-line tail for its last 1, 2 or 3 tiles (the count left after its
full rounds).  The lengths below give partitions of 1 .. 21 tiles, so every
wave of the workgroup meets each tail count, with one partition, with two
merged in the same launch, and with many merged by the merge kernel; the
outputs are compared with the fp64 oracle, and the fused decode step with
the oracle's cache rows."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import scenario
from paged_kv_cache_160_amd.workload_runner import GpuWorkload
from tests._parity import TOL, check_cache_rows, max_err, out_to_f64, say

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 31, 33, 47, 48, 49, 63, 64, 65, 80, 96, 97, 112, 128, 129, 144, 161, 176, 192,
        208, 224, 257, 300, 319, 320, 321]

CASES = [
    # (hq, hkv, d, dtype)
    (4, 2, 64, "f32"),
    (32, 8, 128, "bf16"),
    (16, 16, 128, "f16"),
    (8, 1, 64, "bf16"),
]

# 0: the automatic plan; 176: two partitions for the longest sequence (merged
# in the launch); 48: three tiles per partition (merge kernel)
PARTITIONS = [0, 176, 48]


def _workload(case, seed):
    hq, hkv, d, dtype = case
    return wl.custom_workload(len(LENS), hq, hkv, d, LENS, dtype=dtype, seed=seed,
                              extra_blocks=4 * len(LENS) + 8)


@pytest.mark.parametrize("ps", PARTITIONS)
@pytest.mark.parametrize("case", CASES, ids=[f"{c[3]}-Hq{c[0]}-Hkv{c[1]}-D{c[2]}" for c in CASES])
def test_tail_counts_against_oracle(case, ps):
    say(f"[tail] {case} partition_size {ps}")
    w = _workload(case, seed=29)
    ops = wl.setup_ops(w)
    g = GpuWorkload(w).run(ops)
    seqs = list(range(w.num_seqs))
    tables = g.cache.block_tables(seqs)
    out = out_to_f64(g.cache.decode(g.queries(0), 0, tables=tables, partition_size=ps))
    torch.cuda.synchronize()
    st = scenario.OracleState(w, build_pool=False).run(ops)
    ot, ol = st.tables(seqs)
    assert np.array_equal(tables[0].cpu().numpy(), ot)
    exp = scenario.expected_decode_rows(w, wl.queries(w, 0), seqs, ol)
    err = max_err(out, exp)
    say(f"[tail] max abs err {err:.3e}")
    assert err <= TOL[w.cache_dtype]


@pytest.mark.parametrize("ps", [0, 176])
def test_fused_step_tail_counts_against_oracle(ps):
    """Two fused decode steps (cache write, attention, in-launch merge) over
    the same lengths: outputs against the oracle, pool rows bit for bit."""
    case = (32, 8, 128, "bf16")
    say(f"[tail] fused steps {case} partition_size {ps}")
    w = _workload(case, seed=31)
    w.decode_appends = 2
    ops = wl.setup_ops(w)
    g = GpuWorkload(w).run(ops)
    st = scenario.OracleState(w, build_pool=True).run(ops)
    seqs = list(range(w.num_seqs))
    for step in range(2):
        out = out_to_f64(g.decode_step(seqs, step, partition_size=ps))
        torch.cuda.synchronize()
        st.append_one_each(seqs)
        exp = scenario.expected_decode_paged(st, wl.queries(w, step), seqs)
        err = max_err(out, exp)
        say(f"[tail] step {step} max abs err {err:.3e}")
        assert err <= TOL["bf16"]
    tb, lb = g.cache.alloc.block_tables(seqs)
    for b in seqs:
        check_cache_rows(w, g.cache, 0, b, tb[b].numpy(), int(lb[b]))
