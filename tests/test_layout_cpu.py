"""Host checks of the direct-to-LDS B layout (no GPU).

The B slice of the fast kernels is stored in its natural [k][n] order with the
16-byte chunks of row k XOR-swizzled by f(k) = 4 (k mod 4) ^ 2 (bit 3 of k), and
filled by 1 KiB loads of 16 bytes a lane.  These tests restate the address rule
as the kernel applies it to lanes, waves and load indices, and check that the
image covers the slot exactly once, every LDS row holding its own global row.
"""
import pytest


def f(k):
    return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1))


def image_16(NW, BN, BK):
    RBB = BN * 2
    LPR, RPD = RBB // 16, 64 // (RBB // 16)
    img = {}
    for w in range(NW):
        dg = []
        for e2 in range(2):
            row = []
            for lane in range(64):
                rl, pch = lane // LPR, lane % LPR
                r = 8 * e2 + w * RPD + rl
                row.append((rl, (pch ^ f(r)) * 16))
            dg.append(row)
        for c in range(BK * RBB // 1024 // NW):
            grp = c * NW + w
            e = ((c * NW * RPD) >> 3) & 1
            for lane in range(64):
                rl, colb = dg[e][lane]
                for b in range(16):
                    dst = grp * 1024 + 16 * lane + b
                    assert dst not in img
                    img[dst] = (grp * RPD + rl, colb + b)
    return img


@pytest.mark.parametrize("NW,BN,BK", [(8, 256, 64), (4, 128, 64)])
def test_each_slot_row_holds_its_own_row_once(NW, BN, BK):
    # every LDS row k holds exactly the bytes of global row k, each once
    img = image_16(NW, BN, BK)
    RBB = BN * 2
    for k in range(BK):
        got = sorted(img[k * RBB + x][1] for x in range(RBB))
        assert got == list(range(RBB))
        assert {img[k * RBB + x][0] for x in range(RBB)} == {k}
