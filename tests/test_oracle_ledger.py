"""Pins for the storage formats: the oracle's measured array sizes reproduce the
ledger figures the pages print (tests/golden/ledger.txt holds them with
citations)."""
import pytest

import oracle

N = 64 * 256 * 8          # a whole number of second-level chunks


def test_scale_overhead_bits(golden):
    g = golden("ledger.txt")
    no_dq = oracle.storage_bits_per_weight(N, double_quant_on=False)
    dq = oracle.storage_bits_per_weight(N, double_quant_on=True)
    assert no_dq == g["scale_bits_no_dq"] == 32 / 64
    assert dq == 8 / 64 + 32 / (64 * 256) == 0.126953125
    assert round(dq, 3) == g["scale_bits_dq"]
    assert round(no_dq - dq, 2) == g["scale_bits_saved"]
    # the per-tensor mean adds one float32 per tensor, invisible at model scale
    with_mean = oracle.storage_bits_per_weight(N, include_mean=True)
    assert with_mean - dq == pytest.approx(32 / N)
    # codes: 4 bits per weight, two per byte
    assert oracle.storage_bits_per_weight(N, include_codes=True) - dq == 4.0


def test_65b_budget(golden):
    g = golden("ledger.txt")
    n = g["n_65b"]
    bits_dq = oracle.storage_bits_per_weight(N, include_codes=True)
    bits_no_dq = oracle.storage_bits_per_weight(N, double_quant_on=False, include_codes=True)
    assert n * 16 / 8 / 1e9 == g["gb_65b_16bit"]
    assert n * 4 / 8 / 1e9 == g["gb_65b_4bit"]
    assert round(n * bits_dq / 8 / 1e9, 1) == g["gb_65b_4bit_dq"]
    assert round(n * (bits_dq - 4) / 8 / 1e9) == g["gb_65b_scales_dq"]
    assert round(n * (bits_no_dq - 4) / 8 / 1e9, 1) == g["gb_65b_scales_no_dq"]
    assert round(n * (bits_no_dq - bits_dq) / 8 / 1e9) == g["saving_65b_gb"]


def test_7b_ledger(golden):
    g = golden("ledger.txt")
    n = g["n_7b"]
    gb16, gb4 = n * 16 / 8 / 1e9, n * 4 / 8 / 1e9
    assert gb16 == g["gb_7b_16bit"] and gb4 == g["gb_7b_4bit"]
    assert n * 32 / 8 / 1e9 == g["gb_7b_fp32"] and n * 8 / 8 / 1e9 == g["gb_7b_1byte"]
    # the 4-bit figure is 3.5 decimal GB, i.e. 3.26 GiB (GB = 1e9 bytes, GiB = 2^30)
    assert round(n * 4 / 8 / 2 ** 30, 2) == 3.26
    t16, t4 = gb16 + g["other_gb"], gb4 + g["other_gb"]
    assert (t16, t4) == (g["total_16bit_gb"], g["total_4bit_gb"])
    assert round(t16 / t4, 2) == g["ratio_6gb_other"]
    assert round(t16 / t4, 3) == g["ratio_6gb_other_3dp"]
    assert round((gb16 + 20) / (gb4 + 20), 3) == g["ratio_20gb_other"]


def test_lora_parameter_count(golden):
    g = golden("ledger.txt")
    h, o, r = int(g["lora_h"]), int(g["lora_o"]), int(g["lora_r"])
    assert oracle.lora_param_count(h, o, r) == g["lora_params"]
    assert h * o == g["full_params"]
    assert h * o // oracle.lora_param_count(h, o, r) == g["lora_ratio"]
