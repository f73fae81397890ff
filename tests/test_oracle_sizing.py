"""Pins for the oracle's sizing formulas: the worked values the pages print
(tests/golden/sizing_worked_examples.json, each entry with its citation)."""
import json
import os

import pytest

from oracle import sizing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sizing_worked_examples.json")
DATA = json.load(open(GOLDEN, encoding="utf-8"))


@pytest.mark.parametrize("ex", DATA["examples"], ids=[e["id"] for e in DATA["examples"]])
def test_worked_sizing_values(ex):
    v = sizing.kv_cache_bytes(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["seq_len"],
                              ex["batch"], ex["bytes_per_elem"]) / ex["scale"]
    step = 10.0 ** -ex["decimals"]
    assert ex["printed"] <= v + 1e-12 < ex["printed"] + step, (ex["id"], v)


def test_per_token_bytes_exact():
    # "KV Cache 和 vLLM" §1.3 spells the per-token product out: 40 x 2 x 4096 x 2 bytes
    assert sizing.kv_cache_bytes(40, 32, 128, 1, 1, 2) == 40 * 2 * 4096 * 2 == 655360


def test_gqa_quarter():
    # 32 -> 8 KV heads cuts the cache to a quarter ("企业官网建设流程全解析" §2.2)
    assert sizing.kv_cache_bytes(32, 8, 128, 4096, 1, 2) * 4 == sizing.kv_cache_bytes(32, 32, 128, 4096, 1, 2)


def test_fp8_halves():
    # FP8 takes one byte per element ("KV Cache优化实战" §2.1)
    assert sizing.kv_cache_bytes(32, 8, 128, 4096, 16, 1) * 2 == sizing.kv_cache_bytes(32, 8, 128, 4096, 16, 2)


@pytest.mark.parametrize("ex", DATA["utilisation"], ids=[e["id"] for e in DATA["utilisation"]])
def test_prealloc_utilisation(ex):
    assert sizing.prealloc_utilisation(ex["lengths"], ex["max_len"]) == pytest.approx(ex["expected"])


def test_paged_utilisation_closed_form():
    assert sizing.paged_utilisation([16, 32]) == 1.0
    assert sizing.paged_utilisation([1]) == 1 / 16
    assert sizing.paged_utilisation([17, 40]) == pytest.approx(57 / 80)
