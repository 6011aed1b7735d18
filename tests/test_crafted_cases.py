"""CPU checks that the hand-built code sets in crafted.py reach the branches they
are built for (the GPU tests that use them rely on it): the guard case has every
row maximum at or above 2^18 and uses many levels; the tie-window case has one key
per row at y' in [-1 - 1.7e-4, -1] (exact level 0) in a unit whose every level is
0, after a move of the running maximum."""
import numpy as np

import crafted


def test_tie_window_case(orc):
    cfg, z, info = crafted.tie_window_case(orc)
    assert -1.00017 <= info["y"] <= -1.0
    r = orc.attention(cfg, z, dumps=True)
    pc = r["pcode"]
    assert np.all(pc[:, info["key"]] == -8)
    assert np.all(pc[:, 128:192] == -8)                      # the unit's levels are all 0
    assert np.all((pc[:, 0:128] > -8).sum(axis=1) > 0)        # earlier steps add to O
    assert np.all((pc[:, 192:256] > -8).sum(axis=1) > 0)      # and so does the last one
    # the running maximum moved in step 1 (A 470 > 400): the final m is 470 c
    assert np.all(r["m"] == np.float32(np.float32(470) * np.float32(info["c"])))


def test_guard_case(orc):
    cfg, z = crafted.guard_case(orc)
    r = orc.attention(cfg, z, dumps=True)
    assert r["m"].min() >= 2.0 ** 18
    levels = np.unique(r["pcode"].astype(int) + 8)
    assert len(levels) >= 5 and 0 in levels and 15 in levels
