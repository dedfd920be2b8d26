"""Accounting formulas against the numbers the pages print (tests/golden/accounting_page_numbers.json)."""
import json
import os

import pytest

from grouped_gemm_top_amd import accounting as acc

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting_page_numbers.json")))


def test_lora_params_per_expert_projection():
    g = G["lora_params_per_expert_projection"]
    assert acc.lora_params(g["m"], g["n"], g["r"]) == g["value"]


def test_lora_fraction():
    g = G["lora_fraction_of_projection"]
    assert acc.lora_fraction(g["m"], g["n"], g["r"]) == pytest.approx(g["approx"], rel=g["rtol"])


def test_dense_mlp_example():
    g = G["dense_mlp_example"]
    assert acc.lora_params(g["m"], g["n"], g["r"]) == pytest.approx(g["lora_approx"], rel=g["rtol"])
    assert g["m"] * g["n"] == pytest.approx(g["full_approx"], rel=g["rtol"])
    assert acc.lora_fraction(g["m"], g["n"], g["r"]) == pytest.approx(g["fraction_approx"], rel=g["rtol"])


def test_peft_delta_elements():
    g = G["peft_delta_elements"]
    assert acc.peft_delta_elements(g["E"], g["m"], g["n"]) == pytest.approx(g["approx"], rel=g["rtol"])


def test_memory_crossovers():
    g = G["memory_crossover_unsloth"]
    assert acc.split_memory_crossover(g["E"], g["m"], g["k"]) == g["value"]
    g = G["memory_crossover_rank"]
    assert acc.split_memory_crossover_rank(g["E"], g["m"], g["n"], g["k"], g["r"]) == g["value"]


def test_compute_crossover_formula_and_printed_value():
    g = G["compute_crossover"]
    v = acc.compute_crossover(g["E"], g["m"], g["n"], g["k"], g["r"])
    assert v == pytest.approx(g["formula_value_approx"], rel=g["rtol"])
    # the printed ~16K is E*m/(2k), the m = n approximation of the same formula
    assert g["E"] * g["m"] / (2 * g["k"]) == g["printed"]


def test_flop_formula_matches_the_sum_of_its_gemms():
    s, m, n, E, k, r = 4096, 2048, 768, 128, 8, 16
    f = acc.gemm_flops(s, m, n, E, k, r)
    P = s * k
    # forward: gate_up + down + router
    assert f["fwd"] == f["gate_up_fwd"] + f["down_fwd"] + f["router_fwd"]
    # backward dX GEMMs plus the four LoRA-gradient products per projection
    lora_grads = 2 * P * r * (2 * m + 2 * n) + 2 * P * r * (n + m)
    assert f["bwd"] == f["gate_up_bwd_dx"] + f["down_bwd_dx"] + lora_grads + 2 * s * k * m
    assert round(f["total"] / 1e9, 1) == 647.3
