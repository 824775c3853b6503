"""The planner against measured timings (profiles/planner_sweep.json, written by
bench.py --plan-table from bench.py --plan-sweep runs on MI355X): for the 18 dense
DeepSeek-V3-like shapes, the 10 masked decode cases and the 18 shapes in the TN layout,
the plan the library chooses (256 CUs, unlimited workspace) was measured, and is within
5% of the fastest measured plan of that case. No GPU needed."""
import json
import os

import pytest

import moe_grouped_gemm_fp32_amd as fg

TABLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles", "planner_sweep.json")
DATA = json.load(open(TABLE))


@pytest.fixture(autouse=True)
def cus256():
    fg.set_num_cus(256)
    yield
    fg.set_num_cus(0)


@pytest.mark.parametrize("case", sorted(DATA["dense"]))
def test_dense_plan_within_5_percent_of_best(case):
    M, N, K = (int(x) for x in case.split(","))
    c = fg.query_config(fg.KIND_DENSE, M, N, K, workspace_bytes=1 << 40)
    key = "%dx%d s%d f%d" % (c["block_m"], c["block_n"], c["split_k"], c["full_tiles"] if c["split_k"] > 1 else 0)
    tab = DATA["dense"][case]
    assert key in tab, f"{case}: chosen plan {key} was not measured"
    best = min(tab.values())
    assert tab[key] <= 1.05 * best, f"{case}: {key} {tab[key]} us vs best {best} us"


@pytest.mark.parametrize("case", sorted(DATA["masked"]))
def test_masked_plan_within_5_percent_of_best(case):
    G, N, K = (int(x) for x in case.split(","))
    c = fg.query_config(fg.KIND_MASKED, 4096, N, K, G, expected_m=256, workspace_bytes=1 << 40)
    key = "%dx%d s%d" % (c["block_m"], c["block_n"], c["split_k"])
    tab = DATA["masked"][case]
    assert key in tab, f"masked {case}: chosen plan {key} was not measured"
    best = min(tab.values())
    assert tab[key] <= 1.05 * best, f"masked {case}: {key} {tab[key]} us vs best {best} us"


@pytest.mark.parametrize("case", sorted(DATA["layout"]))
def test_layout_plan_within_5_percent_of_best(case):
    M, N, K = (int(x) for x in case.split(","))
    c = fg.query_config(fg.KIND_LAYOUT, M, N, K, workspace_bytes=1 << 40)
    key = "%dx%d s%d" % (c["block_m"], c["block_n"], c["split_k"])
    tab = DATA["layout"][case]
    assert key in tab, f"layout {case}: chosen plan {key} was not measured"
    best = min(tab.values())
    assert tab[key] <= 1.05 * best, f"layout {case}: {key} {tab[key]} us vs best {best} us"


def test_table_covers_every_case():
    assert len(DATA["dense"]) == 18 and len(DATA["masked"]) == 10 and len(DATA["layout"]) == 18
