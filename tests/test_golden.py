"""Stored expectations: the pages' fixed facts and the oracle's regression record."""

import json
import os

import numpy as np

from workloads import preset

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pages_facts_consistent_with_workloads():
    facts = json.load(open(os.path.join(HERE, "pages_facts.json")))
    for a, g, tau in facts["expected_acceptance_length"]["cases"]:
        # the cases are the printed closed form evaluated at the listed points
        assert abs((1 - a ** (g + 1)) / (1 - a) - tau) < 1e-9
    dopt = {G: D for G, D in facts["attention_gemm_m"]["cases"]}
    assert preset("g8_kv32k_D15").draft_len == dopt[8]
    assert preset("g32_kv128k_D3_greedy").draft_len == dopt[32]


def test_oracle_matches_its_stored_record():
    from tests.golden.make_golden import build
    rec = json.load(open(os.path.join(HERE, "tiny_oracle.json")))
    now = build()
    assert now["stochastic"] == rec["stochastic"]
    assert now["greedy"] == rec["greedy"]
    np.testing.assert_allclose(now["attention"]["sum"], rec["attention"]["sum"], rtol=1e-12)
    np.testing.assert_allclose(now["attention"]["sum_sq"], rec["attention"]["sum_sq"], rtol=1e-12)
    for (ix, v), (ix2, v2) in zip(now["attention"]["samples"], rec["attention"]["samples"]):
        assert ix == ix2
        np.testing.assert_allclose(v, v2, rtol=1e-12, atol=1e-15)
