"""Bound on the number of matrix-core k-steps a head layout can have.

The allocation kernel cuts every width group (widths descending, each group's storage
positions consecutive) into segments of at most 8 positions and packs the segments, in
storage order, into k-steps of 4 segments that draw on at most two groups.  The decode
kernel sizes its LDS operand area for D/32 + 3 k-steps (5, 7 and 11 for head dims 64, 128
and 256) and keeps the first 8 in registers, so the bound below is load-bearing: this test
re-derives it from the packing rule over every possible sequence of group segment counts.

A group of m positions (m even, m >= 2) has ceil(m / 8) segments, so a layout with G groups
and segment counts c_1..c_G needs sum(8 c_g - 6) <= head_dim positions.
"""

from __future__ import annotations

import functools
import itertools

import pytest


def ksteps(counts) -> int:
    """k-steps produced by the packing rule for groups with the given segment counts."""
    ks, slot, ga, gb = -1, 4, -1, -1
    for g, c in enumerate(counts):
        for _ in range(c):
            if slot == 4 or (g != ga and g != gb and gb >= 0):
                ks, slot, ga, gb = ks + 1, 0, g, -1
            elif g != ga and gb < 0:
                gb = g
            slot += 1
    return ks + 1


def max_ksteps(head_dim: int) -> int:
    """Largest k-step count over all layouts of head_dim (dynamic programme over groups)."""

    # state between groups: (slot used in the open k-step, groups in it); value: k-steps so far
    @functools.lru_cache(maxsize=None)
    def best(groups_left: int, budget: int, slot: int, ngrp: int) -> int:
        # largest number of k-steps still to open with groups_left more groups (>= 0 of them)
        out = 0
        if groups_left == 0:
            return 0
        for c in range(1, 17 * 2):
            need = 8 * c - 6
            if need > budget:
                break
            opened, s, n = 0, slot, ngrp
            for i in range(c):
                if s == 4 or (i == 0 and n == 2):
                    opened, s, n = opened + 1, 0, 1
                elif i == 0:
                    n += 1
                s += 1
            out = max(out, opened + best(groups_left - 1, budget - need, s, n))
        return out

    return max(best(g, head_dim, 4, 0) for g in range(1, 9))


def test_packing_rule_matches_a_direct_simulation():
    for counts in itertools.product(range(1, 6), repeat=3):
        segs = [(g, i) for g, c in enumerate(counts) for i in range(c)]
        # direct restatement: open a k-step when it is full or a third group would enter it
        ks, members = [], None
        for g, _ in segs:
            if members is None or len(members[1]) == 4 or (g not in members[0] and len(members[0]) == 2):
                members = ({g}, [g])
                ks.append(members)
            else:
                members[0].add(g)
                members[1].append(g)
        assert ksteps(counts) == len(ks)


def layouts(head_dim: int, groups: int, prefix=()):
    """Every sequence of segment counts of `groups` groups that fits head_dim positions."""
    used = sum(8 * c - 6 for c in prefix)
    if len(prefix) == groups:
        yield prefix
        return
    c = 1
    while used + 8 * c - 6 + 2 * (groups - len(prefix) - 1) <= head_dim:
        yield from layouts(head_dim, groups, prefix + (c,))
        c += 1


@pytest.mark.parametrize("head_dim", [64, 128])
def test_dynamic_programme_matches_brute_force(head_dim):
    brute = max(ksteps(c) for g in range(1, 9) for c in layouts(head_dim, g))
    assert brute == max_ksteps(head_dim)


@pytest.mark.parametrize("head_dim", [64, 128, 256])
def test_kstep_bound_used_by_the_decode_kernel(head_dim):
    assert max_ksteps(head_dim) == head_dim // 32 + 3
