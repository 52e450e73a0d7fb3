"""Host check of the lane bookkeeping behind the D = 64 row sums of the
attention kernel (no GPU): the packed P register that feeds the PV product
is reused as the B operand of a 16x16x32 matrix product against a constant
0/1 selector, and every result register a lane receives must be the sum of
p over the keys of that lane's own query.

Layouts (gfx950 matrix instructions, wave64):
  * P register (B operand of the 32x32x16 PV product): lane l holds 8
    consecutive keys 8 (l // 32) + j, j = 0..7, of query l % 32 (one 16-key
    step of the tile).
  * 16x16x32 product: lane l supplies A[l % 16][8 (l // 16) + j] and
    B[8 (l // 16) + j][l % 16], and receives D[4 (l // 16) + i][l % 16],
    i = 0..3.
  * Selector value of lane l (the same expression as the kernel):
    1 if bit 2 of (l % 16) equals bit 0 of (l // 16), else 0.
"""
import numpy as np


def _selector(lane: int) -> float:
    return 1.0 if (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) else 0.0


def _rowsum_via_16x16x32(p: np.ndarray) -> np.ndarray:
    """p[query, key] for 32 queries x 16 keys -> the 4 result registers of
    each lane, shape [64, 4]."""
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    for lane in range(64):
        for j in range(8):
            k = 8 * (lane // 16) + j
            A[lane % 16, k] = _selector(lane)
            # the P register's element j of this lane: key 8 (l // 32) + j of query l % 32
            B[k, lane % 16] = p[lane % 32, 8 * (lane // 32) + j]
    D = A @ B
    out = np.zeros((64, 4))
    for lane in range(64):
        for i in range(4):
            out[lane, i] = D[4 * (lane // 16) + i, lane % 16]
    return out


def test_every_result_register_holds_the_lanes_own_row_sum():
    rng = np.random.default_rng(7)
    for _ in range(5):
        p = rng.random((32, 16))
        got = _rowsum_via_16x16x32(p)
        want = p.sum(axis=1)
        for lane in range(64):
            np.testing.assert_allclose(got[lane], want[lane % 32], rtol=1e-12, atol=0)


def test_selector_is_needed():
    """An all-ones selector mixes queries n and n + 16 (the check above is
    not vacuous)."""
    rng = np.random.default_rng(8)
    p = rng.random((32, 16))
    B = np.zeros((32, 16))
    for lane in range(64):
        for j in range(8):
            B[8 * (lane // 16) + j, lane % 16] = p[lane % 32, 8 * (lane // 32) + j]
    D = np.ones((16, 32)) @ B
    assert not np.allclose(D[0, 0], p[0].sum())
    assert np.allclose(D[0, 0], p[0].sum() + p[16].sum())
