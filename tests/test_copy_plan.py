"""Host checks of the in-tile copy schedule (sync_protocols_amd/csrc/fg_plan.hpp),
compiled for the CPU with g++ from the same header the kernel includes.

For every shape: each list's items visit each of its tiles exactly once; the
lead slabs are exactly the gathered rows [0, 2048 * lead) that every workgroup
copies first; the non-lead rows of each list are dealt to its items in order,
each row exactly once; and every row is copied by an item of an earlier round
than the first item that reads its slab ("PCIe sync protocols" §6: a consumer
never waits on work scheduled after it), so the copy never waits on the
compute it feeds. A planted mistake (a consumer scheduled in the copier's own
round) is caught by the same check."""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "sync_protocols_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, os.path.join(HERE, "plan_driver.cpp"), "-o", exe],
                   check=True)
    return exe


def group_shape(per_list, n_tn):
    """GN and GS as the compute role picks them."""
    gn = 1
    while gn * 2 <= min(8, per_list) and n_tn % (gn * 2) == 0:
        gn *= 2
    return max(1, per_list // gn), gn


def run_plan(exe, n_slabs, half_last, per_list, n_tn):
    gs, gn = group_shape(per_list, n_tn)
    out = subprocess.run([exe, str(n_slabs), str(half_last), str(per_list), str(n_tn), str(gs), str(gn)],
                         check=True, capture_output=True, text=True).stdout
    lists, items = {}, {}
    for line in out.splitlines():
        f = line.split()
        if f[0] == "L":
            lists[int(f[1])] = dict(ns=int(f[2]), lead=int(f[3]), rows=int(f[4]))
        else:
            x, j, tile, c0, c1 = map(int, f[1:])
            items.setdefault(x, []).append((j, tile, c0, c1))
    return lists, items


def gathered_row(n_slabs, x, lead, rho):
    k = lead + rho // 256
    return 256 * (x + 8 * k) + rho % 256


def check_plan(lists, items, n_slabs, half_last, per_list, n_tn, shift_consumers=0):
    lead_rows = set()
    max_rows = 0
    for x in range(8):
        L = lists[x]
        ns, ld, R = L["ns"], L["lead"], L["rows"]
        its = items.get(x, [])
        assert [j for j, *_ in its] == list(range(ns * n_tn))
        tiles = [t for _, t, _, _ in its]
        want = sorted((x + 8 * k) * n_tn + c for k in range(ns) for c in range(n_tn))
        assert sorted(tiles) == want, f"list {x}: items do not visit each tile once"
        # slab rows
        for k in range(ns):
            s = x + 8 * k
            rows = 128 if (half_last and s == n_slabs - 1) else 256
            if k < ld:
                lead_rows.update(range(256 * s, 256 * s + rows))
        # first round reading each slab
        first_round = {}
        for j, t, _, _ in its:
            s = t // n_tn
            r = j // per_list + shift_consumers
            first_round[s] = min(first_round.get(s, r), r)
        # the copy ranges partition [0, R) in item order
        pos = 0
        for j, t, c0, c1 in its:
            assert c0 == pos and c1 >= c0, f"list {x} item {j}: range [{c0}, {c1}) after {pos}"
            pos = c1
            max_rows = max(max_rows, c1 - c0)
            if c1 > c0:
                r = j // per_list
                assert (r + 1) * per_list <= len(its), f"list {x} item {j}: copies in a partial round"
                for rho in range(c0, c1):
                    g = gathered_row(n_slabs, x, ld, rho)
                    s = g // 256
                    assert s % 8 == x and (s - x) // 8 >= ld, "a non-lead row of this list"
                    assert first_round[s] > r, (f"list {x}: row {g} copied in round {r}, "
                                                f"read from round {first_round[s]}")
        assert pos == R, f"list {x}: {pos} of {R} non-lead rows copied"
    lead = max(lists[x]["lead"] for x in range(8))
    m_pad = 256 * n_slabs - (128 if half_last else 0)
    assert lead_rows == set(range(min(m_pad, 2048 * lead))), "lead rows are the prefix copied first"
    return max_rows


def test_plan_large_share(driver):
    # 8 x 4096 rows, K = N = 8192: 128 slabs, 32 workgroups per XCD, 32 column tiles
    lists, items = run_plan(driver, 128, 0, 32, 32)
    m = check_plan(lists, items, 128, 0, 32, 32)
    assert all(lists[x]["lead"] == 1 for x in range(8))
    assert m <= 32


def test_plan_tp_share(driver):
    # 4 x 2048 rows, N = 4096: 32 slabs, 16 column tiles: two lead slabs per list
    lists, items = run_plan(driver, 32, 0, 32, 16)
    m = check_plan(lists, items, 32, 0, 32, 16)
    assert all(lists[x]["lead"] == 2 for x in range(8))
    assert m == 16


def test_plan_random_shapes(driver):
    rng = np.random.default_rng(5)
    for _ in range(60):
        n_slabs = int(rng.integers(1, 300))
        half = int(rng.integers(0, 2))
        per_list = int(rng.choice([1, 2, 4, 8, 9, 16, 17, 25, 32]))   # grid / 8 for grids of 8 to 256
        n_tn = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        lists, items = run_plan(driver, n_slabs, half, per_list, n_tn)
        m = check_plan(lists, items, n_slabs, half, per_list, n_tn)
        # a compute item's share goes to its 8 waves, one row per lane
        assert m <= 8 * 64, (n_slabs, per_list, n_tn, m)


def test_plan_check_has_teeth(driver):
    # the same plan read as if every consumer ran one round earlier must fail:
    # the copy of the first group is then due in its own round
    lists, items = run_plan(driver, 128, 0, 32, 32)
    with pytest.raises(AssertionError):
        check_plan(lists, items, 128, 0, 32, 32, shift_consumers=-1)
