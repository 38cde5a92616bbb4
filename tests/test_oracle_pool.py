"""Pin of the oracle's append scatter (CPU): scattered rows read back through
the pinned logical gather sit at the positions their destinations name, for
every KV head; a later row wins; every other byte is unchanged; out-of-range
destinations raise.  Planted mistakes in copies of the scatter must fail
(JustVugg/colibri pull 372, Summary: the new rows arrive in one packed upload
and a scatter kernel writes them into their pages)."""

import numpy as np
import pytest

from oracle import pool_model
from oracle_checks import check_scatter


@pytest.mark.parametrize("P,rb", [(16, 144), (48, 272), (64, 512)])
def test_scatter_pinned_by_gather(P, rb):
    check_scatter(pool_model.scatter_rows, pool_model.gather_rows, P=P, rb=rb, seed=P)


def _planted(mistake):
    def scatter(pool, blocks, slots, rows):
        out = pool.copy()
        nb, H, P, rb = out.shape
        for i in range(rows.shape[0]):
            b, s = int(blocks[i]), int(slots[i])
            if not (0 <= b < nb and 0 <= s < P):
                raise IndexError("out of range")
        order = range(rows.shape[0] - 1, -1, -1) if mistake == "first_wins" else range(rows.shape[0])
        for i in order:
            b, s = int(blocks[i]), int(slots[i])
            if mistake == "slot_plus_one":
                s = min(s + 1, P - 1)
            heads = [0] if mistake == "head0_only" else range(H)
            for h in heads:
                src = (H - 1 - h) if mistake == "heads_swapped" else h
                out[b, h, s, :] = rows[i, src, :]
        return out
    return scatter


@pytest.mark.parametrize("mistake", ["slot_plus_one", "head0_only", "heads_swapped", "first_wins"])
def test_scatter_mistakes_fail_the_pin(mistake):
    with pytest.raises(AssertionError):
        check_scatter(_planted(mistake), pool_model.gather_rows)


def test_planted_scatter_without_mistake_passes():
    check_scatter(_planted(None), pool_model.gather_rows)
