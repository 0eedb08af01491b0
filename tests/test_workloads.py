"""Seeded workload generation and byte/FLOP accounting (CPU only)."""

import json
import math
import os

import numpy as np
import pytest

import workloads
from workloads import CONFIGS, make_inputs, round_to_storage

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def test_page_byte_figures():
    figs = json.load(open(GOLDEN))
    s = figs["score_matrix_n2048_fp16"]
    assert workloads.score_matrix_bytes(s["n"], s["itemsize"]) == s["bytes"] == 8 * 2 ** 20
    t = figs["score_tile_64x64_fp32"]
    assert t["rows"] * t["cols"] * t["itemsize"] == t["bytes"] == 16 * 2 ** 10
    for row in figs["naive_to_tiled_bandwidth_reduction"]["rows"]:
        pct = 100 * (1 - row["tiled_gbps"] / row["naive_gbps"])
        assert abs(pct - row["reduction_pct"]) < 0.6, row


def test_headline_accounting():
    w = workloads.get(workloads.HEADLINE)
    assert (w.B, w.H, w.N, w.D, w.dtype, w.causal) == (1, 32, 2048, 64, "f16", False)
    assert workloads.flops(w) == 4 * 32 * 2048 ** 2 * 64
    assert workloads.min_bytes(w) == 32 * 2 ** 20
    causal = w.with_(causal=True)
    assert workloads.flops(causal) == workloads.flops(w) / 2


def test_five_workloads():
    assert len(workloads.ORDER) == 5
    assert len(CONFIGS) == 5 + len(workloads.PAGE_TABLE)
    for w in CONFIGS.values():
        assert math.isclose(w.scale, 1 / math.sqrt(w.D))
    # the second page's comparison shapes: 32 heads, D = 128, N = 512 and 1024
    assert [(workloads.get(n).H, workloads.get(n).D, workloads.get(n).N) for n in workloads.PAGE_TABLE] == \
        [(32, 128, 512), (32, 128, 1024)]
    seeds = [w.seed for w in CONFIGS.values()]
    assert len(set(seeds)) == len(seeds)


def test_deterministic_and_distinct_seeds():
    w = workloads.get("ragged_b2h8n1000d96_f16_uniform_head").with_(N=64)
    a, b = make_inputs(w), make_inputs(w)
    for n in "qkv":
        assert np.array_equal(a[n], b[n])
    c = make_inputs(w.with_(seed=w.seed + 1))
    assert not np.array_equal(a["q"], c["q"])


def test_uniform_head_and_distributions():
    w = workloads.get("ragged_b2h8n1000d96_f16_uniform_head")
    x = make_inputs(w)
    k = x["k"]
    assert (k[0, 0] == k[0, 0, :1]).all()
    assert not (k[0, 1] == k[0, 1, :1]).all()
    q = x["q"].view(np.float16).astype(np.float64)
    assert abs(q.mean()) < 0.01 and abs(q.std() - 1) < 0.01
    w4 = workloads.get("long_prefill_causal_b1h16n8192d128_f16_sigma3").with_(H=1, N=512)
    x4 = make_inputs(w4)
    q4 = x4["q"].view(np.float16).astype(np.float64)
    v4 = x4["v"].view(np.float16).astype(np.float64)
    assert abs(q4.std() - 3) < 0.05
    assert v4.min() >= -1 and v4.max() <= 1 and abs(v4.std() - 1 / math.sqrt(3)) < 0.01


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82), (1 + 2 ** -8 + 2 ** -20, 0x3F81),
    (-2.5, 0xC020), (3.140625, 0x4049),
])
def test_bf16_round_to_nearest_even(x, bits):
    assert int(round_to_storage(np.array([x], dtype=np.float32), "bf16")[0]) == bits


def test_f16_round_to_nearest_even():
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0], dtype=np.float32)
    assert list(round_to_storage(x, "f16")) == [0x3C00, 0x3C02, 0x7BFF]
