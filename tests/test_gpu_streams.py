"""Decode on a stream other than the current one, with the workspace left to
the binding: the binding allocates it on the launch stream, so memory the
current stream allocates and fills right after the call (while the side
stream's kernels may still run) never lands on it.  Outputs against the
oracle; one and two launches (decode, and the split form)."""
import numpy as np
import pytest
import torch

import workloads as wl
import paged_kv_cache_160_amd as pkv
from oracle import scenario
from paged_kv_cache_160_amd.workload_runner import GpuWorkload
from tests._parity import max_err, out_to_f64, say

pytestmark = pytest.mark.gpu


def _setup():
    lens = [3000, 500, 1200, 2047]
    w = wl.custom_workload(len(lens), 8, 2, 128, lens, dtype="bf16", seed=41)
    ops = wl.setup_ops(w)
    g = GpuWorkload(w).run(ops)
    torch.cuda.synchronize()
    seqs = list(range(w.num_seqs))
    exp = scenario.expected_decode_rows(w, wl.queries(w, 0), seqs, lens)
    return w, g, seqs, exp


def _scribble(nbytes: int):
    # allocations on the current stream, filled at once: had the call's
    # workspace been freed to this stream, these would overwrite it
    return [torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda") for _ in range(4)]


@pytest.mark.parametrize("split", [False, True], ids=["one-call", "split"])
def test_decode_on_side_stream_internal_workspace(split):
    w, g, seqs, exp = _setup()
    c = g.cache
    bt, lens, max_len = c.block_tables(seqs)
    q = g.queries(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = pkv.workspace_size(len(seqs), w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, 128, c.cache_code)
    assert need > 0
    say(f"[stream] side-stream decode, split={split}, workspace {need} bytes")
    with torch.cuda.stream(side):
        out = torch.empty_like(q)
    if split:
        _, ws = pkv.paged_attention_decode_append_partials(out, q, None, None, c.k[0], c.v[0], None, bt, lens,
                                                           max_len, partition_size=128, stream=side)
        pkv.paged_attention_merge_partials(out, lens, w.num_kv_heads, w.max_blocks_per_seq, max_len,
                                           c.cache_code, partition_size=128, workspace=ws, stream=side)
        del ws
    else:
        pkv.paged_attention_decode(out, q, c.k[0], c.v[0], bt, lens, max_len, partition_size=128, stream=side)
    junk = _scribble(need)
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    err = max_err(out_to_f64(out), exp)
    say(f"[stream] max abs err {err:.3e}")
    assert err <= 2e-2
