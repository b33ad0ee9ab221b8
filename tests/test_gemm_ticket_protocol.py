"""CPU simulation of the ticket / ready-list protocol of the one-launch
grouped GEMM (GEMM1 and GEMM2 of a pass in one launch, 128-row tiles).

The protocol, as the kernel states it: the m-tiles are split into 8
contiguous runs, one per group of workgroups.  A workgroup takes one ticket
from its group's counter when it starts.  The group's GEMM1 tickets come
first (n1 per m-tile), then its GEMM2 tickets (n2 per m-tile).  A GEMM1 tile
bumps its m-tile's count when it is done; the tile that completes the count
(n1) appends the m-tile to the group's ready list.  The i-th n2 GEMM2
tickets take the i-th ready m-tile: such a tile polls ready[i] (a bounded
wait) and gives up, reporting MOE_ERR_GEMM_WAIT, when the bound runs out.

This model runs the protocol with random tile durations and a limited
number of workgroups resident at once (dispatched in block order, a new one
starting when one ends, which is all the hardware promises), and checks:
every wait ends without the bound for any residency of one or more; each
GEMM2 tile reads an m-tile only after all n1 GEMM1 tiles of it are done;
every m-tile is read by exactly n2 GEMM2 tiles; and with a zero bound the
tiles that give up are reported and write nothing.
"""

import random

import pytest


def simulate(mv, n1, n2, slots, wait_limit, seed):
    rng = random.Random(seed)
    t1 = mv * n1
    tot = t1 + mv * n2
    ticket = 0
    count = [0] * mv
    ready = [0] * mv            # m-tile + 1, 0 = not yet
    ready_n = 0
    done1 = [False] * mv        # all GEMM1 tiles of the m-tile finished
    reads = [0] * mv
    errors = 0
    running = []                # dicts: kind, m / i, left, spins
    next_block = 0
    steps = 0
    while next_block < tot or running:
        steps += 1
        assert steps < 10_000_000, "no progress: a wait never ended"
        while len(running) < slots and next_block < tot:
            next_block += 1
            t = ticket
            ticket += 1
            if t < t1:
                # GEMM1: bands of up to 8 m-tiles, n-tile by n-tile
                band, r = divmod(t, 8 * n1)
                gm = min(8, mv - band * 8)
                nt, off = divmod(r, gm)
                running.append(dict(kind=1, m=band * 8 + off, left=rng.randint(1, 20)))
            else:
                i = (t - t1) // n2
                running.append(dict(kind=2, i=i, m=None, left=rng.randint(1, 12), spins=0))
        wg = rng.choice(running)
        if wg["kind"] == 1:
            wg["left"] -= 1
            if wg["left"] == 0:
                m = wg["m"]
                count[m] += 1
                if count[m] == n1:
                    done1[m] = True
                    ready[ready_n] = m + 1
                    ready_n += 1
                running.remove(wg)
        else:
            if wg["m"] is None:
                if ready[wg["i"]]:
                    wg["m"] = ready[wg["i"]] - 1
                    assert done1[wg["m"]], "GEMM2 read an m-tile before its GEMM1 tiles ended"
                else:
                    wg["spins"] += 1
                    if wait_limit is not None and wg["spins"] > wait_limit:
                        errors += 1          # MOE_ERR_GEMM_WAIT, rows not written
                        running.remove(wg)
                continue
            wg["left"] -= 1
            if wg["left"] == 0:
                reads[wg["m"]] += 1
                running.remove(wg)
    return dict(reads=reads, errors=errors, count=count)


@pytest.mark.parametrize("slots", [1, 2, 5, 64])
@pytest.mark.parametrize("mv,n1,n2", [(1, 4, 4), (9, 4, 4), (18, 4, 1), (3, 1, 8)])
def test_every_wait_ends_and_reads_follow_writes(mv, n1, n2, slots):
    for seed in range(20):
        r = simulate(mv, n1, n2, slots, wait_limit=None, seed=seed)
        assert r["errors"] == 0
        assert r["count"] == [n1] * mv
        assert r["reads"] == [n2] * mv


def test_bounded_wait_reports_and_writes_nothing():
    # one resident workgroup: the GEMM2 tiles only start once every GEMM1
    # tile has ended, so even a zero bound never gives up
    r = simulate(6, 4, 4, 1, wait_limit=0, seed=1)
    assert r["errors"] == 0 and r["reads"] == [4] * 6
    # many resident workgroups and a zero bound: GEMM2 tiles that find their
    # m-tile not ready give up, each reported, and only the others read
    gave_up = 0
    for seed in range(50):
        r = simulate(6, 4, 4, 48, wait_limit=0, seed=seed)
        assert r["errors"] + sum(r["reads"]) == 6 * 4
        gave_up += r["errors"]
    assert gave_up > 0
