"""Pins for the HBM trip-count model of the two loop orders (CPU only).

The closed forms in ``workloads.traffic_q_outer`` / ``traffic_kv_outer`` are
checked against a brute-force walk of the two loop nests that adds up the
size of every tile each loop iteration moves (ragged edges included), and
against the statements of the pages: in the Q-outer order Q is read once, O
and L are written once, K and V are read once per query block (twice for
two blocks), and nothing else crosses; in one tile both orders move the
same bytes.
"""
import itertools

import pytest

import workloads


def walk_q_outer(n, d, Br, Bc, elem, stat=4):
    rd = dict.fromkeys(("Q", "K", "V", "O", "L"), 0)
    wr = dict(rd)
    for i in range(0, n, Br):
        rows = min(Br, n - i)
        rd["Q"] += rows * d * elem
        for j in range(0, n, Bc):
            keys = min(Bc, n - j)
            rd["K"] += keys * d * elem
            rd["V"] += keys * d * elem
        wr["O"] += rows * d * elem
        wr["L"] += rows * stat
    return rd, wr


def walk_kv_outer(n, d, Bc, Br, elem, groups, acc=4, stat=4):
    rd = dict.fromkeys(("Q", "K", "V", "O_acc", "m_l", "O", "L"), 0)
    wr = dict(rd)
    per = -(-n // groups)
    bounds = [(g * per, min(n, (g + 1) * per)) for g in range(groups) if g * per < n]
    for (a, e) in bounds:
        for j in range(0, n, Bc):
            keys = min(Bc, n - j)
            rd["K"] += keys * d * elem
            rd["V"] += keys * d * elem
            last = j + Bc >= n
            for i in range(a, e, Br):
                rows = min(Br, e - i)
                rd["Q"] += rows * d * elem
                if j > 0:
                    rd["O_acc"] += rows * d * acc
                    rd["m_l"] += 2 * rows * stat
                if last:
                    wr["O"] += rows * d * elem
                    wr["L"] += rows * stat
                else:
                    wr["O_acc"] += rows * d * acc
                    wr["m_l"] += 2 * rows * stat
    return rd, wr


@pytest.mark.parametrize("n,d,Br,Bc,elem", itertools.product([1, 63, 64, 65, 200, 256],
                                                              [8, 64], [32, 64], [64], [2, 4]))
def test_q_outer_closed_form_matches_walk(n, d, Br, Bc, elem):
    rd, wr = walk_q_outer(n, d, Br, Bc, elem)
    t = workloads.traffic_q_outer(n, d, Br, elem)
    assert {k: v[0] for k, v in t.items()} == rd
    assert {k: v[1] for k, v in t.items()} == wr


@pytest.mark.parametrize("n,d,Bc,groups,elem", itertools.product([1, 63, 64, 65, 200, 256],
                                                                  [8, 128], [32, 64], [1, 2, 3],
                                                                  [2]))
def test_kv_outer_closed_form_matches_walk(n, d, Bc, groups, elem):
    rd, wr = walk_kv_outer(n, d, Bc, 32, elem, groups)
    t = workloads.traffic_kv_outer(n, d, Bc, elem, groups=min(groups, n))
    assert {k: v[0] for k, v in t.items()} == rd
    assert {k: v[1] for k, v in t.items()} == wr


def test_two_blocks_read_k_and_v_twice():
    # [KV]: with two query blocks K and V are read twice; Q once; O, L written once
    t = workloads.traffic_q_outer(128, 16, 64, 4)
    assert t["K"][0] == t["V"][0] == 2 * 128 * 16 * 4
    assert t["Q"] == (128 * 16 * 4, 0) and t["O"] == (0, 128 * 16 * 4) and t["L"] == (0, 128 * 4)


def test_one_tile_orders_agree():
    # a single tile in each direction: nothing is carried between tiles
    a = workloads.traffic_total(workloads.traffic_q_outer(64, 32, 64, 2))
    b = workloads.traffic_total(workloads.traffic_kv_outer(64, 32, 64, 2))
    assert a == b


def test_kv_outer_carries_grow_with_tiles():
    # every extra key tile adds one read and one write of O_acc, m and l per row
    n, d = 1024, 64
    t1 = workloads.traffic_kv_outer(n, d, 64, 2)
    t2 = workloads.traffic_kv_outer(n, d, 128, 2)
    assert t1["O_acc"][0] == 15 * n * d * 4 and t2["O_acc"][0] == 7 * n * d * 4
    assert t1["Q"][0] == 16 * n * d * 2
