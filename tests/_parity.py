"""Shared helpers for the GPU parity tests: tolerances, pool read-back and the
comparison of GPU cache contents with the oracle's expectation."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import workloads as wl
from oracle import kv_formats

# Maximum absolute error of decode outputs against the fp64 oracle: 1e-5 for
# fp32 inputs, 2e-2 for bf16 / f16 / fp8 inputs.
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2, "fp8_e4m3": 2e-2, "fp8_e5m2": 2e-2, "int8_int4": 2e-2}

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def say(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def tol_for(w: wl.Workload) -> float:
    return TOL[w.cache_dtype]


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits_of_values(vals: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bits of values exactly representable in ``dtype``."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(TORCH[dtype])
    return t.view(torch.int32 if dtype == "f32" else torch.int16).numpy()


def slots_for(table_row, length: int, bs: int = 16) -> np.ndarray:
    t = np.arange(length)
    return np.asarray(table_row, dtype=np.int64)[t // bs] * bs + t % bs


def gather_gpu_rows(pool: torch.Tensor, slots: np.ndarray) -> torch.Tensor:
    """Rows [n, Hkv, D] stored at the given slots of a device pool
    ``[num_blocks, Hkv, bs, D]`` (raw dtype)."""
    bs = pool.shape[2]
    s = torch.from_numpy(slots).to(pool.device)
    return pool[s // bs, :, s % bs, :]


def check_cache_rows(w: wl.Workload, cache, layer: int, seq: int, table_row, length: int) -> None:
    """Bit-exact: the GPU pool holds, at the slots the oracle's tables give for
    positions 0..L-1, the rows the oracle expects (copies, or e4m3 codes and
    scales from the oracle's quantiser for quantised formats)."""
    slots = slots_for(table_row, length, w.block_size)
    k_rows = wl.kv_rows(w, seq, "k", length)
    v_rows = wl.kv_rows(w, seq, "v", length)
    gk = gather_gpu_rows(cache.k[layer], slots).cpu()
    gv = gather_gpu_rows(cache.v[layer], slots).cpu()
    k_elem, v_elem = kv_formats.FORMATS[w.cache_dtype]
    if kv_formats.is_quantised(k_elem):
        for rows, got, scale_pool, elem in ((k_rows, gk, cache.k_scale[layer], k_elem),
                                            (v_rows, gv, cache.v_scale[layer], v_elem)):
            codes, scales = kv_formats.quantise(rows, elem)
            assert np.array_equal(got.view(torch.uint8).numpy(), codes), f"seq {seq}: {elem} codes differ"
            s = torch.from_numpy(slots).to(scale_pool.device)
            gs = scale_pool[s // w.block_size, :, s % w.block_size].cpu().numpy()
            assert np.array_equal(gs.view(np.uint32), scales.view(np.uint32)), f"seq {seq}: scales differ"
    else:
        view = torch.int32 if w.cache_dtype == "f32" else torch.int16
        assert np.array_equal(gk.view(view).numpy(), bits_of_values(k_rows, w.cache_dtype)), f"seq {seq}: K differs"
        assert np.array_equal(gv.view(view).numpy(), bits_of_values(v_rows, w.cache_dtype)), f"seq {seq}: V differs"


def max_err(got: np.ndarray, exp: np.ndarray) -> float:
    assert got.shape == exp.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - exp))) if got.size else 0.0
