"""The host-side schedule against the step ranges the page states for its default run
(fixture tests/golden/schedule_default_run.json) and the sweep offsets' properties."""
import json
import os

import pytest

from sampled_softmax_cross_amd import schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_default_run.json")


def test_default_run_matches_the_stated_ranges():
    g = json.load(open(GOLDEN))
    a, b = g["stage2"]
    # stages 0 and 1 share [0, a) (their split does not change P); stage 2 is [a, b);
    # the batch taper and the extension follow
    for split in (1, 340, a - 1):
        bounds = [(0, split), (split, a), (a, b), (b, b + 15), (b + 15, g["total_steps"])]
        got = [schedule.candidate_count(bounds, s) for s in range(g["total_steps"])]
        for r in g["expected"]:
            assert set(got[r["first"]:r["last"] + 1]) == {r["P"]}, (split, r)


def test_equal_parts_and_custom_tables():
    bounds = [(0, 10), (10, 19)]
    table = {1: (1, 2, 3)}
    assert [schedule.candidate_count(bounds, s, table) for s in range(10, 19)] == [1, 1, 1, 2, 2, 2, 3, 3, 3]
    assert schedule.candidate_count(bounds, 5, table) == 0          # stage 0 not listed
    assert schedule.candidate_count(bounds, 19, table) == 3         # past the end: last stage
    assert schedule.stage_of(bounds, 25) == 1


@pytest.mark.parametrize("V,world", [(50304, 8), (50304, 3), (7, 7), (1000, 1)])
def test_rank_offsets(V, world):
    offs = [schedule.rank_offset(V, r, world) for r in range(world)]
    assert offs[0] == 0 and all(0 <= o < V for o in offs)
    assert offs == sorted(offs) and len(set(offs)) == world
    assert max(b - a for a, b in zip(offs, offs[1:] + [V])) - min(b - a for a, b in zip(offs, offs[1:] + [V])) <= 1
    with pytest.raises(ValueError):
        schedule.rank_offset(V, world, world)
