"""Host model of the grouped GEMM's K-major weight path (each W_e stored
[K, N], read for the dgrad products of the backward without a transpose).

The kernel loads a weight stage as BK rows of BN features with LDS-DMA
(lane L of a 1 KiB block lands at byte 16 L; 64-byte segments XOR-swizzled
by row & 3) and reads MFMA fragments with ds_read_b64_tr_b16, whose lane
layout (lane o of a 16-lane group gets column o of the group's 4 rows, when
4 lanes per row address 4 columns each) was measured on the GPU. This model
re-runs both address computations on a numbered matrix and checks that every
lane's fragment holds the 8 consecutive k of its feature that
v_mfma_f32_32x32x16_bf16 expects, and that no load leaves W_e.
"""
import numpy as np
import pytest

BK, BN, TN, WN = 64, 256, 4, 128
ROWB_T = BN * 2  # bytes per row of a K-major stage


def dma_stage(W, n0, k0, TM):
    """LDS bytes of one weight stage (2-byte cells, -1 = unwritten) and the
    largest element index read."""
    K, N = W.shape
    a_bytes = 64 * TM * 128
    LB = BN // 32
    lds = np.full(a_bytes + BK * ROWB_T, -1, dtype=np.int64)
    top = 0
    for wave in range(4):
        for i in range(LB):
            dst = a_bytes + (wave * LB + i) * 1024
            for L in range(64):
                kr = (wave * LB + i) * 2 + (L >> 5)
                p = (L & 31) >> 2
                col = min(n0 + 32 * (p ^ (kr & 3)) + 8 * (L & 3), N - 8) - n0
                boff = (kr * N + col) * 2
                assert boff < 2 ** 32
                g = k0 * N + n0 + boff // 2
                top = max(top, g + 8)
                lds[dst + 16 * L: dst + 16 * L + 16: 2] = W.flat[g:g + 8]
    return lds, a_bytes, top


def tr_read(lds, addrs):
    """ds_read_b64_tr_b16 over 64 lane addresses: 4 values per lane."""
    out = []
    for g in range(4):
        B = [[lds[addrs[16 * g + i] + 2 * m] for m in range(4)] for i in range(16)]
        out += [[B[4 * q + o // 4][o % 4] for q in range(4)] for o in range(16)]
    return out


@pytest.mark.parametrize("N,K,n0,k0,TM", [(1024, 4096, 768, 4032, 4), (4096, 1024, 256, 0, 3),
                                          (192, 128, 0, 64, 1), (320, 64, 256, 0, 2)])
def test_k_major_weight_fragments(N, K, n0, k0, TM):
    W = np.arange(K * N, dtype=np.int64).reshape(K, N)
    lds, a_bytes, top = dma_stage(W, n0, k0, TM)
    assert top <= K * N
    for wn in range(2):
        for it in range(TN):
            for s in range(4):
                halves = []
                for h in range(2):
                    addrs = []
                    for lane in range(64):
                        hi = lane >> 5
                        rb = ((8 * hi + ((lane & 15) >> 2)) * ROWB_T + 32 * ((lane >> 4) & 1)
                              + 8 * (lane & 3))
                        wo = a_bytes + rb + 64 * ((4 * wn + it) ^ ((lane >> 2) & 3))
                        addrs.append(wo + s * 16 * ROWB_T + 2048 * h)
                    halves.append(tr_read(lds, addrs))
                for lane in range(64):
                    l5, hi = lane & 31, lane >> 5
                    n = n0 + wn * WN + 32 * it + l5
                    if n >= N:
                        continue  # columns past N are never stored
                    got = halves[0][lane] + halves[1][lane]
                    want = [W[k0 + 16 * s + 8 * hi + j, n] for j in range(8)]
                    assert got == want, (wn, it, s, lane)
