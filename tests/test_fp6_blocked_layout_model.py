"""CPU model of the stage-blocked E2M3 workspace that the FP4-rate NVFP4 path
hands to the FP6-rate kernel, restated from the two sides' index arithmetic:

* writer (requant_nvfp4_e2m3_kernel, stage-blocked): lane b of the output
  writes 24 bytes at 24 b; b counts the four 32-element blocks of a stage of
  a row, the eight rows of a group, the stages, then the groups; padding rows
  past the last (rows rounded up to 8) get zero codes;
* reader (gemm_mxfp6_kernel's load_op, stage-blocked): wave-load L of a
  256-row tile covers rows 8L .. 8L+7; lane i fetches the 12-byte piece
  p = (i % 8) ^ (i / 8) ^ (L % 8) of row 8L + i / 8 at offset
  96 (i / 8) + 8 L lda + 768 ks + 12 p from the tile's first row, inside a
  buffer resource of the tile's rows rounded up to 8 (lda = 96 nk bytes).

Every fetch of a real row must find that row's stage ks, piece p; every fetch
past the resource must be a padding row past the operand; and the resource
of every tile must lie inside the padded code array the workspace holds."""
import numpy as np
import pytest

TM, NW = 256, 8
LOADS_OP = TM // 8 // NW          # wave-loads per wave and operand of a stage


def writer(rows: int, K: int) -> np.ndarray:
    """Padded code array: entry [b] = (row, block-in-row) whose 24 bytes lane
    b writes, (-1, -1) for a padding row."""
    kbr, nk = K // 32, K // 128
    rows8 = -(-rows // 8) * 8
    out = np.full((rows8 * kbr, 2), -1, np.int64)
    for b in range(rows8 * kbr):
        t = b >> 5
        g = t // nk
        row = 8 * g + ((b >> 2) & 7)
        if row < rows:
            out[b] = (row, 4 * (t - g * nk) + (b & 3))
    return out


def reader_check(rows: int, K: int, layout: np.ndarray) -> int:
    """Replay every operand fetch of every tile and stage; returns the number
    of in-bounds fetches checked."""
    lda, nk = K * 6 // 8, K // 128
    rows8 = -(-rows // 8) * 8
    assert layout.shape[0] * 24 == rows8 * lda
    checked = 0
    for m0 in range(0, rows, TM):
        res = ((min(rows - m0, TM) + 7) & ~7) * lda          # the tile's buffer resource
        base = m0 * lda
        assert base + res <= rows8 * lda
        for ks in range(nk):
            for L in range(NW * LOADS_OP):
                for lane in range(64):
                    piece = (lane & 7) ^ (lane >> 3) ^ (L & 7)
                    off = 96 * (lane >> 3) + 8 * L * lda + 768 * ks + 12 * piece
                    row = m0 + 8 * L + (lane >> 3)
                    if off + 12 > res:
                        assert off >= res, "a fetch straddles the resource end"
                        assert row >= rows, f"row {row} of {rows} fetched out of bounds"
                        continue
                    # piece p holds elements 16 p .. 16 p + 15 of the stage: half p % 2 of the
                    # 24-byte block 4 ks + p / 2 of the row
                    a = base + off
                    assert a % 12 == 0
                    blk, rem = divmod(a, 24)
                    want_row, want_blk = (row, 4 * ks + piece // 2) if row < rows else (-1, -1)
                    assert tuple(layout[blk]) == (want_row, want_blk), (rows, K, m0, ks, L, lane)
                    assert rem == 12 * (piece % 2)
                    checked += 1
    return checked


@pytest.mark.parametrize("rows,K", [(256, 128), (300, 640), (2301, 512), (7, 256), (263, 1152)],
                         ids=lambda v: str(v))
def test_blocked_writer_and_reader_agree(rows, K):
    layout = writer(rows, K)
    n = reader_check(rows, K, layout)
    rows8 = -(-rows // 8) * 8
    # every real row's every block is fetched (each block as two 12-byte pieces) by exactly the tiles' loads
    assert n == 2 * rows8 * (K // 32)


def test_blocked_stage_is_contiguous():
    """Stage ks of rows 8g .. 8g+7 is 768 contiguous bytes, rows in order."""
    rows, K = 24, 384
    layout = writer(rows, K)
    nk = K // 128
    for g in range(rows // 8):
        for ks in range(nk):
            unit = layout[(g * nk + ks) * 32:(g * nk + ks + 1) * 32]
            assert [tuple(x) for x in unit] == [(8 * g + r, 4 * ks + q) for r in range(8) for q in range(4)]


def test_row_major_reader_would_straddle_lines():
    """Why the blocked order: in the row-major layout a wave-load's eight
    96-byte row pieces touch 12 128-byte lines on average (half of them
    straddle two lines), in the blocked one six whole lines."""
    K = 8192
    lda = K * 6 // 8
    lines_rm, lines_blk = [], []
    for ks in range(K // 128):
        rm = {(r * lda + 96 * ks + o) // 128 for r in range(8) for o in (0, 95)}
        lines_rm.append(len(rm))
        blk = {(768 * ks + o) // 128 for o in range(0, 768, 4)}
        lines_blk.append(len(blk))
    assert np.mean(lines_rm) == 12 and set(lines_blk) == {6}
