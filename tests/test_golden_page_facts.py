"""The work model behind every roofline figure, pinned to numbers the pages print."""
import json
import os

import pytest

from head_attention_flash_amd import accounting as acc

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))["facts"]


def _approx(got, want, rel):
    assert abs(got - want) <= rel * abs(want), f"{got} vs printed {want} (rel {rel})"


@pytest.mark.parametrize("fact", FACTS, ids=[f["id"] for f in FACTS])
def test_page_fact(fact):
    i = fact["id"]
    if i == "band_keys_per_query":
        S, w = fact["S"], fact["window"]
        # interior queries: the pair count per query away from both ends
        assert acc.band_pairs(S, w) - acc.band_pairs(S - 1, w) == fact["value"]
        assert 2 * w + 1 == fact["value"]
    elif i == "one_head_kv_bytes":
        _approx(fact["S"] * fact["D"] * fact["bytes_per_el"], fact["approx"], fact["rel"])
    elif i == "dit_score_elements_per_call":
        _approx(fact["heads"] * acc.band_pairs(fact["S"], -1) * fact["branches"], fact["approx"], fact["rel"])
    elif i == "dit_useful_matmul_ms_at_peak":
        flops = fact["calls"] * acc.diff_flops(1, fact["heads"], fact["S"], -1)
        _approx(flops / fact["peak_flops"] * 1e3, fact["approx_ms"], fact["rel"])
    elif i == "decoder_projection_MB":
        _approx(fact["tokens"] * fact["channels"] * fact["bytes_per_el"] / 1e6, fact["approx_MB"], fact["rel"])
    elif i == "band_kernel_floor_ms_per_clip":
        per_block = acc.diff_bytes(1, fact["heads"], fact["tokens"])
        _approx(fact["blocks"] * per_block / fact["bw"] * 1e3, fact["approx_ms"], fact["rel"])
    elif i == "sdxl_l1_scores_MB":
        _approx(fact["heads"] * fact["S"] * fact["S"] * fact["bytes_per_el"] / 1e6, fact["approx_MB"], fact["rel"])
    else:
        pytest.fail(f"unknown fact {i}")


def test_band_pairs_brute_force():
    for S in (1, 2, 5, 17, 18, 35, 36, 100):
        for w in (-1, 0, 1, 3, 17, 40):
            brute = sum(1 for p in range(S) for j in range(S) if w < 0 or abs(p - j) <= w)
            assert acc.band_pairs(S, w) == brute
