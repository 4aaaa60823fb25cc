"""Cut planner (host logic, no GPU): the event-graph simulation that scores
candidate designs and the search over cut sets of a decode step.  Pinned by the
worked example the pages print, by brute force over every cut set, and by cases
whose best design is known in closed form."""
import itertools
import json
import os
import random

import pytest

import persistent_megakernel_02_amd.mk as mk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "planner_worked_example.json")


def test_worked_example_serial_and_overlap():
    """Chunk ready at 20 ms; serially the rest of production and decoding take 4
    and 6 ms with a 0.1 ms switch; side by side on split resources 6 and 8 ms with
    a 0.2 ms switch: first release at 30.1 ms serially, 28.2 ms overlapped."""
    g = json.load(open(GOLDEN))
    s, o = g["serial"], g["overlap"]
    ser = mk.event_sim([dict(duration=g["chunk_ready_ms"]),
                        dict(duration=s["producer_ms"], deps=[0]),
                        dict(duration=s["consumer_ms"], deps=[1], dispatch=s["switch_ms"])])
    ovl = mk.event_sim([dict(duration=g["chunk_ready_ms"]),
                        dict(duration=o["producer_ms"], deps=[0], stream=1),
                        dict(duration=o["consumer_ms"], deps=[0], stream=2, dispatch=o["switch_ms"])])
    assert ser[-1] == pytest.approx(s["first_release_ms"], abs=1e-9)
    assert ovl[-1] == pytest.approx(o["first_release_ms"], abs=1e-9)
    assert ovl[-1] < ser[-1]  # each part slower, released earlier


def test_event_sim_stream_order_and_dependencies():
    # same stream: in order even without a dependency; other streams overlap
    f = mk.event_sim([dict(duration=3), dict(duration=2), dict(duration=5, stream=1), dict(duration=1, deps=[1, 2])])
    assert f == [3.0, 5.0, 5.0, 6.0]
    with pytest.raises(mk.MKError):
        mk.event_sim([dict(duration=1, deps=[1]), dict(duration=1)])  # dependency on a later task
    with pytest.raises(mk.MKError):
        mk.event_sim([dict(duration=-1)])


def _brute(layer, head, launch, refill):
    """Best step time over every set of launch starts (regions: layers, then the head)."""
    L = len(layer)
    regions = list(layer) + [head]
    best = None
    for k in range(L + 1):
        for cut in itertools.combinations(range(1, L + 1), k):
            starts = [0] + list(cut)
            t = 0.0
            for j, a in enumerate(starts):
                b = starts[j + 1] if j + 1 < len(starts) else L + 1
                t += launch + refill[a] + sum(regions[a:b])
            if best is None or t < best[0] - 1e-9:
                best = (t, list(cut))
    return best


@pytest.mark.parametrize("L", [3, 6, 11, 17])
def test_plan_matches_brute_force(L):
    """The planner's choice (simulated enumeration up to 16 layers, dynamic
    programming beyond) has the brute-force optimum's step time."""
    rng = random.Random(L)
    for trial in range(4):
        layer = [rng.uniform(20, 60) for _ in range(L)]
        refill = [rng.uniform(-15, 10) for _ in range(L + 1)]  # launch durations stay positive
        refill[0] = 0.0
        launch, head = rng.uniform(0, 15), rng.uniform(50, 100)
        want_t, _ = _brute(layer, head, launch, refill)
        got = mk.plan_cuts(layer, launch, head, refill)
        assert got["predicted_us"] == pytest.approx(want_t, rel=1e-12, abs=1e-9)
        # the returned cuts reproduce the score
        starts = [0] + got["cuts"]
        regions = layer + [head]
        t = sum(launch + refill[a] + sum(regions[a:(starts[j + 1] if j + 1 < len(starts) else L + 1)])
                for j, a in enumerate(starts))
        assert t == pytest.approx(got["predicted_us"], rel=1e-12)


def test_plan_single_launch_when_cuts_only_cost():
    """With a positive launch cost and no refill gain, one launch is best."""
    got = mk.plan_cuts([47.0] * 16, launch_us=8.0, head_us=85.0, refill_us=[5.0] * 17)
    assert got["cuts"] == [] and not got["conventional"]
    assert got["predicted_us"] == pytest.approx(8.0 + 5.0 + 16 * 47.0 + 85.0)
    assert got["single_launch_us"] == got["predicted_us"]


def test_plan_cuts_where_a_launch_start_pays_off():
    """A region that runs faster at a launch start (say, a merged kernel spills
    there) by more than a launch costs gets a cut; the others do not."""
    refill = [0.0] * 17
    refill[9] = -25.0
    got = mk.plan_cuts([47.0] * 16, launch_us=10.0, head_us=85.0, refill_us=refill)
    assert got["cuts"] == [9]
    assert got["predicted_us"] == pytest.approx(got["single_launch_us"] - 15.0)


def test_plan_prefers_the_conventional_path_only_when_faster():
    costs = dict(layer_us=[47.0] * 16, launch_us=8.0, head_us=85.0)
    assert mk.plan_cuts(**costs, conventional_us=1082.0)["conventional"] is False
    got = mk.plan_cuts(**costs, conventional_us=500.0)
    assert got["conventional"] is True and got["predicted_us"] == 500.0


def test_plan_rejects_bad_tables():
    with pytest.raises(mk.MKError):
        mk.plan_cuts([], 1.0, 1.0)
    with pytest.raises(mk.MKError):
        mk.plan_cuts([1.0], -1.0, 1.0)
    with pytest.raises(mk.MKError):  # a launch with a negative service time
        mk.plan_cuts([1.0, 1.0], 1.0, 1.0, refill_us=[0.0, -5.0, 0.0])
