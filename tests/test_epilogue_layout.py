"""Host model of the grouped GEMM's staged bf16 epilogue (epilogue_staged in
ffn_bf16.hip).

After the K loop, lane (l5, hi) of a wave holds, for each 32-token slab j,
32-feature tile i and group q, the 4 features 32 i + 8 q + 4 hi + {0..3} of
token l5 of the slab. It writes them (8 bytes) into the wave's 8 KiB
staging area at row l5, 16-byte chunk (4 i + q) ^ (l5 & 15), half hi; lane
(rq, rc) then reads, for g = 0..7, row 4 g + rq at chunk rc ^ (row & 15) and
stores those 16 bytes as features 8 rc .. 8 rc + 7 of that token. This model
replays both address computations on numbered values and checks that every
store gets exactly the features it claims, that the writes cover the 8 KiB
once, and that the reads and writes keep to the bank spread the kernel's
comment states (a ds_read_b128 of 64 lanes touches each 16-byte bank group
of a 256-byte window four times, the minimum for 1 KiB; a ds_write_b64 pass
of a (i, q) pair twice, the minimum for 512 bytes).
"""
from collections import Counter

TN = 4  # 32-feature tiles per wave


def write_address(l5, hi, i, q):
    return l5 * 256 + 8 * hi + (((4 * i + q) ^ (l5 & 15)) << 4)


def read_address(rq, rc, g):
    r = 4 * g + rq
    return r * 256 + ((rc ^ (r & 15)) << 4)


def test_staged_slab_round_trip():
    lds = {}
    for lane in range(64):
        l5, hi = lane & 31, lane >> 5
        for i in range(TN):
            for q in range(4):
                a = write_address(l5, hi, i, q)
                assert 0 <= a < 8192 and a % 8 == 0
                for v in range(4):  # 4 bf16 values, 2 bytes each
                    key = a + 2 * v
                    assert key not in lds, "two writes to one LDS byte"
                    lds[key] = (l5, 32 * i + 8 * q + 4 * hi + v)  # (token, feature)
    assert len(lds) == 8192 // 2
    for lane in range(64):
        rq, rc = lane >> 4, lane & 15
        for g in range(8):
            a = read_address(rq, rc, g)
            assert a % 16 == 0
            got = [lds[a + 2 * v] for v in range(8)]
            row = 4 * g + rq
            assert got == [(row, 8 * rc + v) for v in range(8)], (lane, g)


def test_staged_slab_banks():
    # reads: 64 lanes x 16 bytes; count the lanes per 16-byte bank group
    for g in range(8):
        groups = Counter((read_address(lane >> 4, lane & 15, g) % 256) // 16 for lane in range(64))
        assert set(groups.values()) == {4}
    # writes of one (i, q): 64 lanes x 8 bytes
    for i in range(TN):
        for q in range(4):
            slots = Counter((write_address(lane & 31, lane >> 5, i, q) % 256) // 8 for lane in range(64))
            assert set(slots.values()) == {2}
