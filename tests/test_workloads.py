"""The seeded input generators: determinism, shapes, and exact representability."""
import numpy as np
import pytest
import torch

import workloads


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_shapes(cid):
    w = workloads.make_workload(cid)
    assert len(w.context_lens) == w.num_seqs
    assert w.num_q_heads % w.num_kv_heads == 0
    assert sorted(w.free_order.tolist()) == list(range(w.num_blocks))
    assert max(w.context_lens) <= 16 * w.max_blocks_per_seq


def test_pool_sizes_and_lengths():
    assert workloads.make_workload(2).num_blocks == 4506
    assert workloads.make_workload(5).num_blocks == 72090
    w3 = workloads.make_workload(3)
    assert min(w3.context_lens) >= 1 and max(w3.context_lens) <= 2048
    w4 = workloads.make_workload(4)
    assert all(1500 + 64 <= L <= 1500 + 512 for L in w4.context_lens)
    assert workloads.make_workload(1).context_lens == [1, 16, 17, 40]


def test_streams_deterministic_and_independent():
    w = workloads.make_workload(3)
    a = workloads.kv_rows(w, 5, "k")
    b = workloads.kv_rows(w, 5, "k")
    assert np.array_equal(a, b)
    assert a.shape == (w.context_lens[5], 32, 128)
    # a prefix of a longer draw equals the shorter draw
    assert np.array_equal(workloads.kv_rows(w, 5, "k", 3), a[:3])
    assert not np.array_equal(workloads.kv_rows(w, 6, "k", 3), a[:3])


def test_prefix_rows_shared():
    w = workloads.make_workload(4)
    k0 = workloads.kv_rows(w, 0, "k")
    k3 = workloads.kv_rows(w, 3, "k")
    assert np.array_equal(k0[:1500], k3[:1500])
    assert not np.array_equal(k0[1500:1564], k3[1500:1564])


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_values_exactly_representable(dtype, tdt):
    x = workloads.random_rows(1, 1, (1000,), dtype)
    t = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    assert np.array_equal(t, x)


def test_churn_script_respects_capacity():
    w = workloads.make_workload(3)
    live, used = [], 0
    for op, arg in w.churn_ops:
        if op == "alloc":
            live.append(arg)
            used += arg
            assert used <= w.num_blocks
        else:
            used -= live.pop(arg)
    assert len(w.churn_release) == len(live)


def test_workload5_golden_matches_generator():
    # the stored expectations of the long fp8 workload were written by
    # tests/golden/make_workload5_expected.py from these very inputs
    import json
    import os
    from tests.golden.make_workload5_expected import input_fingerprint
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "workload5_expected.json")) as f:
        rec = json.load(f)
    w = workloads.make_workload(5)
    assert rec["input_fingerprint"] == input_fingerprint(w)
    out = np.load(os.path.join(here, "workload5_expected.npz"))["out"]
    assert out.shape == (w.num_seqs, w.num_q_heads, w.head_dim) and np.all(np.isfinite(out))
    assert [s["seq"] for s in rec["sequences"]] == list(range(w.num_seqs))
    assert all(s["context_len"] == L for s, L in zip(rec["sequences"], w.context_lens))
