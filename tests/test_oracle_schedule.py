"""Pins of the integer schedule oracle: closed forms, invariants, hand-worked tables."""
import os

import numpy as np
import pytest

from oracle import model
from oracle import schedule as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(tuple(int(v) for v in line.split()))
    return rows


def test_grouped_matches_hand_worked_table():
    for t, tm, tn in _table("grouped_nm5_nn3_G2.txt"):
        assert sch.grouped(t, 5, 3, 2) == (tm, tn)


@pytest.mark.parametrize("nm", range(1, 14))
@pytest.mark.parametrize("nn", [1, 2, 3, 7, 8, 13])
def test_grouped_is_bijection_with_closed_form_ends(nm, nn):
    T = nm * nn
    for G in range(1, nm + 3):
        got = [sch.grouped(t, nm, nn, G) for t in range(T)]
        assert sorted(got) == [(m, n) for m in range(nm) for n in range(nn)]
        if G == 1:  # one tile row per group: row-major
            assert got == [sch.row_major(t, nm, nn) for t in range(T)]
        if G >= nm:  # one group holding every row: column-major
            assert got == [(t % nm, t // nm) for t in range(T)]


def test_grouped_rejects_nonpositive_group():
    with pytest.raises(ValueError):
        sch.grouped(0, 4, 4, 0)


def test_tile_id_spacing_claims_of_the_swizzle_page():
    # Row-major: C(m, n) and C(m+1, n) are num_n_tiles ids apart (128 at N=8192,
    # 256 at N=16384 with BLOCK_N = 64).  Grouped with G = 8: consecutive ids.
    for N, nn_expect in ((8192, 128), (16384, 256)):
        nn = model.cdiv(N, 64)
        assert nn == nn_expect
        nm = model.cdiv(N, 128)
        inv_rm = {sch.row_major(t, nm, nn): t for t in range(nm * nn)}
        inv_g = {sch.grouped(t, nm, nn, 8): t for t in range(nm * nn)}
        for m, n in ((0, 0), (3, 17), (nm - 2, nn - 1)):
            assert inv_rm[(m + 1, n)] - inv_rm[(m, n)] == nn
            if (m + 1) % 8 != 0:
                assert inv_g[(m + 1, n)] - inv_g[(m, n)] == 1


def test_xcd_remap_hand_table_and_permutation():
    for w, r in _table("xcd_remap_n20_x8.txt"):
        assert sch.xcd_remap(w, 20, 8) == r
    for n in range(0, 600):
        got = sorted(sch.xcd_remap(w, n, 8) for w in range(n))
        assert got == list(range(n))
        # each chiplet's round-robin share is one contiguous run
        for x in range(8):
            ids = [sch.xcd_remap(w, n, 8) for w in range(x, n, 8)]
            assert ids == list(range(ids[0], ids[0] + len(ids))) if ids else True


@pytest.mark.parametrize("mode", [sch.PERSISTENT, sch.CROSSTILE])
@pytest.mark.parametrize("remap", [False, True])
def test_persistent_coverage(mode, remap):
    for nm, nn, ks, P in [(5, 7, 3, 4), (8, 8, 1, 64), (3, 3, 0, 2), (20, 49, 2, 256), (4, 4, 5, 100)]:
        s = sch.Schedule(order=sch.GROUPED, group_m=3, mode=mode, num_programs=P, xcd_remap=remap)
        Pe = sch.grid_size(nm * nn, s)
        assert Pe == min(P, nm * nn)
        seen = []
        for p in range(Pe):
            items = sch.program_items(p, nm, nn, ks, s)
            start = sch.xcd_remap(p, Pe) if remap else p
            # k ascending and contiguous per tile; tiles in id order start, start+P, ...
            ksp = max(ks, 1)
            assert len(items) == model.cdiv(nm * nn - start, Pe) * ksp
            for i in range(0, len(items), ksp):
                chunk = items[i:i + ksp]
                assert [c[2] for c in chunk] == list(range(ksp))
                assert len({c[:2] for c in chunk}) == 1
                t = start + (i // ksp) * Pe
                assert chunk[0][:2] == sch.grouped(t, nm, nn, 3)
            seen += items
        assert sorted(seen) == sorted((m, n, k) for m in range(nm) for n in range(nn) for k in range(max(ks, 1)))


def test_crosstile_hand_worked_table():
    s = sch.Schedule(order=sch.ROW_MAJOR, mode=sch.CROSSTILE, num_programs=4)
    got = []
    for p in range(4):
        for it, item in enumerate(sch.program_items(p, 2, 3, 2, s)):
            got.append((p, it) + item)
    assert got == _table("crosstile_nm2_nn3_ks2_P4.txt")


def test_flattened_and_nested_loops_visit_the_same_sequence():
    for order in (sch.ROW_MAJOR, sch.GROUPED):
        a = sch.Schedule(order=order, group_m=4, mode=sch.PERSISTENT, num_programs=7, xcd_remap=True)
        b = sch.Schedule(order=order, group_m=4, mode=sch.CROSSTILE, num_programs=7, xcd_remap=True)
        for p in range(7):
            assert sch.program_items(p, 9, 5, 3, a) == sch.program_items(p, 9, 5, 3, b)


def test_persistent_page_counts():
    # 4096^2 output with 128x64 tiles: 2048 tiles; 340 programs (170 SMs x 2)
    # leave most programs 6 tiles and some 7.
    T = model.cdiv(4096, 128) * model.cdiv(4096, 64)
    assert T == 2048
    s = sch.Schedule(mode=sch.PERSISTENT, num_programs=340)
    counts = [len(sch.program_items(p, 32, 64, 1, s)) for p in range(340)]
    assert min(counts) == 6 and max(counts) == 7
    assert counts.count(7) == 8 == model.tiles_per_program(T, 340)[2]


def test_trace_layout_pads_with_minus_one():
    s = sch.Schedule(order=sch.ROW_MAJOR, mode=sch.CROSSTILE, num_programs=4)
    tr = sch.trace(2 * 64, 3 * 64, 2 * 32, 64, 64, 32, s)
    assert tr.shape == (4 * 4, 5)
    rows = [tuple(r) for r in tr if r[0] >= 0]
    assert rows == _table("crosstile_nm2_nn3_ks2_P4.txt")
    assert (tr[tr[:, 0] < 0] == -1).all() and (tr[:, 0] < 0).sum() == 4


# ---- stream-K split -------------------------------------------------------------------

def test_streamk_hand_worked_table():
    s = sch.Schedule(order=sch.ROW_MAJOR, mode=sch.STREAMK, num_programs=4)
    got = []
    for p in range(4):
        for it, item in enumerate(sch.program_items(p, 2, 3, 3, s)):
            got.append((p, it) + item)
    assert got == _table("streamk_nm2_nn3_ks3_P4.txt")


@pytest.mark.parametrize("nm,nn,ks,P", [(20, 49, 16, 256), (5, 7, 3, 4), (4, 4, 5, 100), (3, 3, 1, 2),
                                        (2, 2, 4, 7), (8, 8, 2, 64), (1, 1, 9, 4), (7, 9, 13, 32)])
@pytest.mark.parametrize("remap", [False, True])
def test_streamk_coverage_and_balance(nm, nn, ks, P, remap):
    s = sch.Schedule(order=sch.GROUPED, group_m=3, mode=sch.STREAMK, num_programs=P, xcd_remap=remap)
    T = nm * nn
    Pe = sch.grid_size(T, s, ks)
    assert Pe == min(P, T * ks)
    split = T % Pe
    whole = T - split
    seen, split_lens = [], []
    for p in range(Pe):
        items = sch.program_items(p, nm, nn, ks, s)
        n_split = len(items) - (len(range(p if not remap else sch.xcd_remap(p, Pe), whole, Pe)) * ks)
        split_lens.append(n_split)
        sk = items[:n_split]
        # a piece is contiguous in (tile id, k) order and no longer than a tile
        assert n_split <= ks
        ids = [(sch.grouped_table(nm, nn, 3).index(it[:2]), it[2]) for it in sk]
        lin = [t * ks + k for t, k in ids]
        assert lin == list(range(lin[0], lin[0] + len(lin))) if lin else True
        assert len({t for t, _ in ids}) <= 2
        # its whole tiles follow, each with all of its K steps in order
        rest = items[n_split:]
        for i in range(0, len(rest), ks):
            assert [c[2] for c in rest[i:i + ks]] == list(range(ks))
        seen += items
    assert sorted(seen) == sorted((m, n, k) for m in range(nm) for n in range(nn) for k in range(ks))
    # piece lengths differ by at most one, longer pieces on higher program indices
    assert max(split_lens) - min(split_lens) <= 1
    assert split_lens == sorted(split_lens)
    assert sum(split_lens) == split * ks


def test_streamk_without_split_is_persistent():
    # whole rounds only (T a multiple of P), or K = 0: nothing is split
    for nm, nn, ks, P in [(4, 4, 3, 8), (4, 4, 0, 5)]:
        a = sch.Schedule(order=sch.GROUPED, group_m=2, mode=sch.STREAMK, num_programs=P, xcd_remap=True)
        b = sch.Schedule(order=sch.GROUPED, group_m=2, mode=sch.PERSISTENT, num_programs=P, xcd_remap=True)
        Pe = sch.grid_size(nm * nn, a, ks)
        if ks == 0:
            assert Pe == min(P, nm * nn)
        for p in range(Pe):
            if ks > 0 or nm * nn % Pe == 0:
                assert sch.program_items(p, nm, nn, ks, a) == sch.program_items(p, nm, nn, ks, b) or ks == 0
