"""Values the pages print (tests/golden/*.json, each citing its passage)."""
import json
import os

import kda_inputs as G

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_prefix_hit_boundary():
    g = _load("p1_worked_hit.json")
    hb = g["hash_block"]
    # the hit is the longest hash-block-aligned boundary within the match
    b = (g["matched_tokens"] // hb) * hb
    assert b == g["hit_boundary"] == g["hit_boundary_in_hash_blocks"] * hb
    assert 0 < b < g["physical_block"] and b % g["physical_block"] != 0
    # the library's hash-block constant and the 8K prefill config use it
    assert G.HASH_BLOCK == hb
    assert g["hit_boundary"] in G.PREFILL_8K.ckpts
    assert all(p % hb == 0 for p in G.PREFILL_8K.ckpts + G.SINGLE_1K.ckpts + G.LONG_1M.ckpts)


def test_state_size_arithmetic():
    g = _load("p1_state_size.json")
    per_req = g["layers"] * g["heads"] * g["d_k"] * g["d_v"] * g["bytes_per_element"]
    assert per_req == 217_055_232
    assert round(per_req / 1e6) == g["stated_state_size_millions"]
    n_ck = g["context"] // g["checkpoint_every"]
    assert n_ck == g["stated_checkpoints"]
    assert n_ck * per_req / 2**30 > g["stated_total_gib_lower_bound"]
    # one head's fp32 state at d = 128 is 64 KiB: the per-head unit of our pool
    assert g["d_k"] * g["d_v"] * 4 == 64 * 1024
