"""CPU model of the LDS layouts the gfx950 kernels stage through, restated
from their addressing: for each layout, the writer (which lane of which
direct-to-LDS wave-load puts which global bytes where) and the reader (which
address each lane reads) are replayed, every read must find the bytes it
wants, and no read may put two distinct dwords in one bank.  Two bank models
are checked, since whether the LDS serves a read 128 or 256 bytes at a time
decides which rows collide: 32 banks of 4 bytes (dword reads 32 lanes a pass,
8-byte reads 16, 16-byte reads 8) and 64 banks (32, 32, 16 lanes).

Layouts:
* chunked MX scale rows (16 bytes per row = 4 E4M3 or 2 E2M1 stages), dwords
  permuted by bits 3-4 of the row (dword reads) or the 8-byte halves by bit 3
  ^ bit 4 (8-byte reads);
* the FP6 kernel's chunk rows (dword reads, like E4M3);
* raw NVFP4 per-stage scale rows (16 bytes, each lane half reading two bytes
  of the k-step's dword), dwords permuted by bits 3-4 of the row;
* operand rows of 128 bytes, 16-byte chunks permuted by (row ^ row / 8) % 8,
  read 16 bytes a lane;
* the FP6 kernel's operand rows: 12-byte pieces landing in 16-byte cells
  under the same permutation, read 12 bytes a lane (taken here in the
  passes of 16-byte reads).
"""
import pytest

TM = TN = 256
MODELS = {"128B": (32, {4: 32, 8: 16, 12: 8, 16: 8}), "256B": (64, {4: 32, 8: 32, 12: 16, 16: 16})}


def banks_ok(addrs, nbytes, model):
    """addrs: per lane, in lane order; each pass covers `per_pass` lanes; no
    bank may serve two distinct dwords within a pass."""
    nbanks, per = MODELS[model]
    per_pass = per[nbytes]
    for p0 in range(0, len(addrs), per_pass):
        seen = {}
        for a in addrs[p0:p0 + per_pass]:
            for d in range(a // 4, (a + nbytes + 3) // 4):
                b = d % nbanks
                if seen.setdefault(b, d) != d:
                    return False
    return True


# ---- chunked MX scale rows ---------------------------------------------------

def chunk_swz(bps, row):
    """Dword XOR of row `row` of the 16-byte chunk rows."""
    return (row >> 3) & 3 if bps == 4 else 2 * (((row >> 3) ^ (row >> 4)) & 1)


def mx_chunk_lds(bps):
    """Writer: portion u of a chunk covers rows u R .. of the concatenated list
    (A rows, then B rows); 16 rows per dword wave-load, lane i landing on
    dword position i % 4 of row i / 4 and fetching dword (i % 4) ^ swz(row)."""
    spc = 16 // bps
    R = (TM + TN) // spc
    lds = {}
    for u in range(spc):
        for row0 in range(u * R, (u + 1) * R, 16):
            for lane in range(64):
                row, pos = row0 + lane // 4, lane % 4
                lds[row * 16 + 4 * pos] = (row, pos ^ chunk_swz(bps, row))
    assert len(lds) == (TM + TN) * 4
    return lds


@pytest.mark.parametrize("bps", [4, 8], ids=["e4m3-dword-reads", "e2m1-8-byte-reads"])
def test_mx_chunk_scale_rows(bps):
    lds = mx_chunk_lds(bps)
    # reader: lane (h, lr) of wave (wm, wn) reads row wm*128 + 32 i + lr (A) or TM + wn*64 + 32 j + lr (B);
    # the lane's base carries 4 swz(row) in bits 2-3, the stage j's byte offset j*bps enters by XOR
    bases = [wm * 128 + 32 * i for wm in range(2) for i in range(4)] + [TM + wn * 64 + 32 * j
                                                                         for wn in range(4) for j in range(2)]
    for base in bases:
        for j in range(16 // bps):
            addrs = []
            for lane in range(64):
                row = base + (lane & 31)
                sa = (row * 16) | (4 * chunk_swz(bps, row))
                a = sa ^ (j * bps)
                addrs.append(a)
                for w in range(bps // 4):           # the stage's dwords, in order
                    assert lds[a + 4 * w] == (row, j * (bps // 4) + w)
            for model in MODELS:
                assert banks_ok(addrs[:32], bps, model), (bps, base, j, model)


def test_unswizzled_chunk_rows_would_conflict():
    """The same reads without the swizzle collide under both models (why it is there)."""
    for bps in (4, 8):
        addrs = [lr * 16 for lr in range(32)]
        assert not banks_ok(addrs, bps, "256B") and not banks_ok(addrs, bps, "128B")


# ---- the FP6 kernel's chunk rows ---------------------------------------------------

def test_fp6_chunk_scale_rows():
    """gemm_mxfp6: 4 stages a chunk, 128 rows a portion, wave w of 8 taking rows
    128 u + 16 w ..; dword position p of row r holds dword p ^ ((r / 8) % 4)."""
    lds = {}
    for u in range(4):
        for w in range(8):
            row0 = u * 128 + 16 * w
            for lane in range(64):
                row, pos = row0 + lane // 4, lane % 4
                lds[row * 16 + 4 * pos] = (row, pos ^ ((row >> 3) & 3))
    for base in [wm * 128 + 32 * i for wm in range(2) for i in range(4)] + [TM + wn * 64 + 32 * j
                                                                             for wn in range(4) for j in range(2)]:
        for j in range(4):
            addrs = []
            for lane in range(32):
                row = base + lane
                a = ((row * 16) | (4 * ((row >> 3) & 3))) ^ (4 * j)
                assert lds[a] == (row, j)
                addrs.append(a)
            for model in MODELS:
                assert banks_ok(addrs, 4, model)


# ---- raw NVFP4 per-stage scale rows -----------------------------------------------

def test_nvfp4_stage_scale_rows():
    """Per-stage dword loads, four lanes a 16-byte row (row = 16 n + lane / 4 of
    the operand's part), lane position `word` fetching dword word ^ ((row / 8) %
    4); each lane half h reads bytes 2h, 2h + 1 of the k-step's dword kk."""
    lds = {}
    for n in range(TM * 16 // 256):
        for lane in range(64):
            d = n * 64 + lane
            row, word = d // 4, d % 4
            lds[row * 16 + 4 * word] = (row, word ^ ((row >> 3) & 3))
    for base in range(0, TM, 32):
        for kk in range(4):
            addrs = []
            for lane in range(64):
                h, lr = lane >> 5, lane & 31
                row = base + lr
                a = (((row * 16) | (4 * ((row >> 3) & 3))) ^ (4 * kk)) + 2 * h
                assert lds[a & ~3] == (row, kk)
                addrs.append(a & ~3)
            for model in MODELS:
                assert banks_ok(addrs[:32], 4, model), (base, kk, model)


# ---- operand rows ----------------------------------------------------------------

def test_operand_chunk_swizzle():
    """128-byte rows, 16-byte chunk c of row r at (c ^ ((r ^ r / 8) % 8)); a
    k-step's fragment read takes chunk 2 kk + h (16-bit and E2M1 operands) of
    rows lr = 0 .. 31: every pass of 16-byte reads covers distinct banks."""
    def swz(r):
        return (r ^ (r >> 3)) & 7
    for base in range(0, 256, 32):
        for kk in range(4):
            addrs = []
            for lane in range(64):
                h, lr = lane >> 5, lane & 31
                row = base + lr
                c = 2 * kk + h
                addrs.append(row * 128 + 16 * (c ^ swz(row)))
            # lanes 0..31 (h = 0) and 32..63 (h = 1) go in separate passes
            for model in MODELS:
                assert banks_ok(addrs[:32], 16, model) and banks_ok(addrs[32:], 16, model), (base, kk, model)


# ---- the FP6 kernel's operand rows ------------------------------------------------

def test_fp6_operand_pieces():
    """gemm_mxfp6: wave-load L (0 .. 31) of an operand's 256 rows puts lane i's
    12 bytes in cell i % 8 of row 8L + i / 8, fetching piece (i % 8) ^ (i / 8) ^
    (L % 8) of that row's stage (so cell c of row r holds piece c ^ swz(r)).
    Lane (h, lr) of wave (wm, wn) reads k-step kk of block blk from base
    (row * 128) | ((swz(lr) << 4) ^ 32 h), XORed with 64 (kk ^ blk % 2), plus
    blk * 4096, and the cell after it (address ^ 16): pieces 4 kk + 2 h and
    4 kk + 2 h + 1 of rows wm * 128 + 32 blk + lr (A, 4 blocks) and
    wn * 64 + 32 blk + lr (B, 2 blocks)."""
    def swz(r):
        return (r ^ (r >> 3)) & 7
    lds = {}
    for L in range(32):
        for i in range(64):
            r, c = 8 * L + i // 8, i % 8
            lds[r * 128 + 16 * c] = (r, (i % 8) ^ (i // 8) ^ (L % 8))
    assert all(piece == (a % 128) // 16 ^ swz(r) for a, (r, piece) in lds.items())
    for nblk, nw, rows_per_wave in ((4, 2, 128), (2, 4, 64)):
        for wv in range(nw):
            for kk in range(2):
                for blk in range(nblk):
                    addrs = []
                    for lane in range(64):
                        h, lr = lane >> 5, lane & 31
                        base = ((wv * rows_per_wave + lr) * 128) | ((swz(lr) << 4) ^ (32 * h))
                        x = (base ^ (64 * (kk ^ (blk & 1)))) + blk * 32 * 128
                        row = wv * rows_per_wave + 32 * blk + lr
                        assert lds[x] == (row, 4 * kk + 2 * h) and lds[x ^ 16] == (row, 4 * kk + 2 * h + 1)
                        addrs.append(x)
                    # the two reads of the fragment (x, then x ^ 16), each in two lane halves
                    for rd in (addrs, [x ^ 16 for x in addrs]):
                        for model in MODELS:
                            assert banks_ok(rd[:32], 12, model) and banks_ok(rd[32:], 12, model), \
                                (nblk, wv, kk, blk, model)

