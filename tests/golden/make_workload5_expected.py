"""Write the expected cache contents and decode outputs of the long-context
fp8 workload (32 sequences x 32768 tokens, 32 query / 8 KV heads, head_dim
128, K/V rows quantised to e4m3 with a float32 scale per (token, head), bf16
queries) for every one of its 32 sequences.

Everything here comes from the oracle and the seeded input generator only:
  * per sequence, SHA-256 digests of the e4m3 codes and float32 scales the
    oracle's quantiser gives for the K and the V rows, in logical order
    ([L][Hkv][D] codes, [L][Hkv] scales): the GPU pool, gathered in the same
    order, must hash to the same values (bit-exact cache write);
  * per sequence, the fp64 decode output over the dequantised rows for the
    queries of step 0.
The oracle takes about a minute per sequence (quantisation dominates), too
slow for a GPU test to run for all 32 sequences, so the values are stored.

    python tests/golden/make_workload5_expected.py [--procs N]

writes tests/golden/workload5_expected.npz (outputs, float64 [32][32][128])
and tests/golden/workload5_expected.json (digests and an input fingerprint).
Pages: "KV Cache优化实战" §3.2-3.3 (fp8 KV with per-token, per-head scales);
"企业官网建设流程全解析" §1.2 (the attention it decodes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402
from oracle import attention, kv_formats  # noqa: E402

WORKLOAD = 5
NPZ = os.path.join(HERE, "workload5_expected.npz")
JSON = os.path.join(HERE, "workload5_expected.json")


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def input_fingerprint(w: wl.Workload) -> str:
    """Digest of the step-0 queries and the first 64 K/V rows of sequences 0
    and 31: a cheap check that the seeded generator still draws these inputs."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(wl.queries(w, 0)).tobytes())
    for b in (0, w.num_seqs - 1):
        for which in ("k", "v"):
            h.update(np.ascontiguousarray(wl.kv_rows(w, b, which, 64)).tobytes())
    return h.hexdigest()


def one_sequence(b: int):
    w = wl.make_workload(WORKLOAD)
    L = w.context_lens[b]
    k_elem, v_elem = kv_formats.FORMATS[w.cache_dtype]
    digests = {}
    values = []
    for which, elem in (("k", k_elem), ("v", v_elem)):
        rows = wl.kv_rows(w, b, which, L)
        codes, scales = kv_formats.quantise(rows, elem)
        digests[which + "_codes"] = sha(codes)
        digests[which + "_scales"] = sha(scales.astype(np.float32).view(np.uint32))
        values.append(kv_formats.dequantise(codes, scales, elem))
    q = wl.queries(w, 0)[b]
    out = attention.attend(q, values[0], values[1], 1.0 / math.sqrt(w.head_dim))
    print(f"[golden] sequence {b}: L={L} done", flush=True)
    return b, L, digests, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    w = wl.make_workload(WORKLOAD)
    B = w.num_seqs
    out = np.zeros((B, w.num_q_heads, w.head_dim), dtype=np.float64)
    seqs = [None] * B
    with ProcessPoolExecutor(max_workers=args.procs) as ex:
        for b, L, digests, o in ex.map(one_sequence, range(B)):
            out[b] = o
            seqs[b] = {"seq": b, "context_len": L, **digests}
    np.savez(NPZ, out=out)
    rec = {
        "workload": w.name, "num_seqs": B, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
        "head_dim": w.head_dim, "cache_dtype": w.cache_dtype, "q_dtype": w.q_dtype,
        "input_fingerprint": input_fingerprint(w),
        "layout": "codes [L][Hkv][D] uint8 and scales [L][Hkv] float32 bits, logical order",
        "written_by": "tests/golden/make_workload5_expected.py (oracle + seeded generator only)",
        "sequences": seqs,
    }
    with open(JSON, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"[golden] wrote {NPZ} and {JSON}", flush=True)


if __name__ == "__main__":
    main()
