"""The stored oracle counts agree with each other (CPU): every per-call
record in calls.json sums the per-frame records of the same frames, a call
that starts a volume creates every block it touches, and the blocks the
calls create add up to the block count at the end of the last call."""
import json
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


CALLS = {k: v for k, v in _load("calls.json").items() if k != "written_by"}


@pytest.mark.parametrize("workload,split", [(w, s) for w, v in CALLS.items() for s in v])
def test_calls_match_frame_counts(workload, split):
    frames = _load(f"{workload}_counts.json")["frames"]
    calls = CALLS[workload][split]
    assert calls[0]["first"] == 0
    for c, nxt in zip(calls, calls[1:] + [None]):
        fr = frames[c["first"]:c["end"]]
        assert c["frames"] == len(fr)
        for k in ("pixels", "points_valid", "voxel_updates"):
            assert c[k] == sum(f[k] for f in fr), k
        if nxt is not None:
            assert nxt["first"] == c["end"]
        before = frames[c["first"] - 1]["blocks_total"] if c["first"] else 0
        assert c["blocks_new"] == fr[-1]["blocks_total"] - before
        assert c["blocks_new"] == sum(f["blocks_new"] for f in fr)
        assert max(f["blocks_touched"] for f in fr) <= c["blocks_touched"] <= sum(f["blocks_touched"] for f in fr)
        assert max(f["voxels_touched"] for f in fr) <= c["voxels_fresh"] + c["voxels_old"] \
            <= sum(f["voxels_touched"] for f in fr)
    first = calls[0]
    assert first["blocks_touched"] == first["blocks_new"] and first["voxels_old"] == 0
