"""The adaptive verify-width controller: its oracle pinned to the pages and to hand-worked
schedules, and the library's controller (host code behind the C-ABI, no GPU needed) against
that oracle, decision by decision."""
import json
import os

import numpy as np
import pytest

from block_drafting_dflash_amd import binding
from oracle.width_controller import WidthController as OracleController

GOLD = os.path.join(os.path.dirname(__file__), "golden", "width_controller_hand.json")


def cases():
    return json.load(open(GOLD))["cases"]


@pytest.mark.parametrize("case", cases(), ids=[c["name"] for c in cases()])
def test_oracle_follows_the_hand_worked_schedules(case):
    w = OracleController(case["depth"], case["ceiling"], case["window"], case["challenge_every"])
    for block, committed, ms in case["rounds"]:
        assert w.width() == block
        w.record(block, committed, ms)
    assert w.incumbent == case["final_incumbent"]
    assert sum(d[3] for d in w.decisions) == case["adoptions"]


def test_oracle_starts_at_the_declared_depth_and_probes_depth_and_ceiling():
    """dflash_round_loop_starts_at_the_configured_depth and
    probed_widths_cover_the_warm_up_depth_and_the_ceiling, as the page names them."""
    for depth, ceiling in [(4, 16), (2, 8), (5, 5), (1, 32)]:
        w = OracleController(depth, ceiling, 3, 2)
        assert w.width() == depth
        assert set(w.probed_widths()) == {depth, ceiling}
    with pytest.raises(ValueError):
        OracleController(8, 4, 1, 1)


def test_oracle_never_leaves_the_two_widths_and_challenges_on_schedule():
    rng = np.random.default_rng(5)
    w = OracleController(4, 16, 5, 3)
    widths = []
    for _ in range(3000):
        b = w.width()
        widths.append(b)
        w.record(b, int(rng.integers(1, b + 2)), float(rng.uniform(0.2, 0.6)) * (1 + b / 16))
    assert set(widths) <= {4, 16}
    # one challenge window per three incumbent windows: a quarter of the windows
    n_windows = len(widths) // 5
    assert len(w.decisions) in (n_windows // 4, n_windows // 4 + 1)


def test_library_controller_follows_the_hand_worked_schedules():
    for case in cases():
        c = binding.WidthController(case["depth"], case["ceiling"], case["window"], case["challenge_every"])
        for block, committed, ms in case["rounds"]:
            assert c.width() == block, case["name"]
            c.record(block, committed, ms)
        st = c.state()
        assert st["incumbent"] == case["final_incumbent"] and st["adoptions"] == case["adoptions"], case["name"]


@pytest.mark.parametrize("seed,depth,ceiling,window,every", [(1, 4, 16, 8, 4), (2, 4, 16, 1, 1), (3, 2, 8, 3, 2),
                                                             (4, 5, 5, 2, 1), (5, 1, 32, 16, 3)])
def test_library_controller_matches_the_oracle(seed, depth, ceiling, window, every):
    """The same random stream of round results through both: the same width before every
    round, the same incumbent rate bit for bit, the same adoptions."""
    rng = np.random.default_rng(seed)
    o = OracleController(depth, ceiling, window, every)
    c = binding.WidthController(depth, ceiling, window, every)
    for r in range(4000):
        b = o.width()
        assert c.width() == b, r
        # acceptance and round time drift over the run so that both widths get adopted
        p = 0.5 + 0.45 * np.sin(r / 300.0)
        k = int(rng.binomial(b, max(0.01, min(0.99, p))))
        ms = float(rng.uniform(0.3, 0.5)) * (1.0 + b / 12.0)
        o.record(b, k + 1, ms)
        c.record(b, k + 1, ms)
        st = c.state()
        if o.incumbent_rate is not None:
            assert st["incumbent_rate"] == o.incumbent_rate
        assert st["incumbent"] == o.incumbent and st["challenging"] == o.challenging
    assert c.state()["adoptions"] == sum(d[3] for d in o.decisions)
    if depth != ceiling and window * every < 200:
        assert c.state()["adoptions"] > 0


def test_library_controller_refuses_bad_records():
    c = binding.WidthController(4, 16, 2, 1)
    L = binding.lib()
    assert L.dflash_width_ctl_record(c.h, 16, 3, 1.0) == 6  # not the width asked for: DFLASH_E_STATE
    assert L.dflash_width_ctl_record(c.h, 4, 0, 1.0) == 3  # no committed token: DFLASH_E_RANGE
    assert L.dflash_width_ctl_record(c.h, 4, 2, 0.0) == 3
    assert c.state()["incumbent_rate"] == -1.0 and c.width() == 4
    h = __import__("ctypes").c_void_p()
    assert L.dflash_width_ctl_create(5, 4, 1, 1, __import__("ctypes").byref(h)) == 3
    assert L.dflash_width_ctl_width(None) == 0
