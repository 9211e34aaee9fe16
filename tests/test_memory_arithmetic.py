"""The pages' memory figures (tests/golden/memory_figures.json, each cited)
against the byte accounting of the formats (CPU only)."""
import json
import os

import pytest

from oracle import memory

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "memory_figures.json")))


def test_bytes_per_param_and_llama_7b():
    g = GOLD["bytes_per_param"]
    for fmt in ("fp16", "int8", "int4"):
        assert memory.weight_bytes_per_param(fmt) == g[fmt]
        assert memory.weight_bytes_per_param(fmt) * g["llama2_7b_params"] / 1e9 == pytest.approx(g["llama2_7b_gb"][fmt])


def test_weight_savings_nominal_and_exact():
    s = GOLD["weight_savings"]
    assert 1 - memory.weight_bytes_per_param("int8") / 2 == s["int8"]
    assert 1 - memory.weight_bytes_per_param("int4") / 2 == s["int4"]
    # with the block constants the saving is a little smaller than the nominal figure
    exact4 = 1 - memory.weight_bytes_per_param("int4", 64) / 2                    # 4.5 bit / param
    exact4dq = 1 - memory.weight_bytes_per_param("int4", 64, nested=True) / 2     # ~4.127 bit / param
    assert exact4 == pytest.approx(0.71875)
    assert exact4dq == pytest.approx(1 - (0.5 + 1 / 64 + 4 / 16384) / 2)
    assert exact4 < exact4dq < s["int4"]


def test_optimizer_state():
    o = GOLD["optimizer_state"]
    b32 = memory.adam_state_bytes_per_param(32)
    b8 = memory.adam_state_bytes_per_param(8)
    assert (b32, b8) == (o["adamw32_bytes_per_param"], o["adamw8bit_bytes_per_param"])
    assert 1 - b8 / b32 == o["saving"]
    assert 7e9 * b32 / 1e9 == o["llama2_7b_gb"]["adamw32"]
    assert 7e9 * b8 / 1e9 == o["llama2_7b_gb"]["adamw8bit"]
    assert 7e9 * (b32 - b8) / 1e9 == o["llama2_7b_gb"]["saved"]
    # with one fp32 absmax per 2048-element block of each moment
    exact = memory.adam_state_bytes_per_param(8, 2048)
    assert exact == pytest.approx(2.00390625) and 1 - exact / b32 == pytest.approx(0.7495117)


def test_savings_table():
    for row in GOLD["savings_table"]["rows"]:
        assert memory.total_saving(row["model"], row["optimizer"]) == pytest.approx(row["total_saving"])


def test_nested_quant_saving():
    bits = memory.nested_saving_bits(64, 256)
    assert bits == pytest.approx(0.373046875)
    assert round(bits, 1) == GOLD["nested_quant"]["extra_saving_bits_per_param"]
