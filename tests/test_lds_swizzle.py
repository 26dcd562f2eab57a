"""CPU model of the K/V tile layout in LDS used by the bf16 attention kernels.

The kernels stage a tile of K and V rows (one key per row, d bf16 values =
ROW bytes) into LDS with global->LDS DMA and read MFMA operands back:

* DMA: wave instruction n writes 1 KB; lane l's 16 bytes land at LDS byte
  n * 1024 + 16 l, i.e. at (key, physical chunk) of the unpadded rows, and
  the lane fetches the logical chunk physical ^ swz(key) of that key.
* K operand (ds_read_b128, S^T = K Q^T on v_mfma_f32_32x32x16_bf16): lane
  (i, h) = (lane % 32, lane // 32) reads key 32 kb + i, logical chunk
  2 ks + h (d values 16 ks + 8 h .. + 7).
* V^T operand (ds_read_b64_tr_b16, O^T += V^T P^T): in each group of 16
  lanes, lane j points at 4 consecutive d values of one of 4 consecutive
  keys; the transposing read hands lane j one d column of those 4 keys.
  Two such reads (keys + 0..3 and + 8..11) give the 8 operand values.

This file rebuilds those address formulas and checks, for d = 128 and
d = 64, that every operand read returns the logical values the MFMA needs
and that no two lanes served in the same LDS cycle touch the same bank
(64 banks of 4 bytes; 16 lanes per cycle for 16-byte reads, 32 lanes for
8-byte reads). The kernel's own counters agree (zero bank-conflict cycles),
but this model pins the layout without a GPU.
"""

import pytest

WAVES = 8
BANKS = 64


def swz_k(row, key):
    return (key & 15) if row == 256 else ((key >> 1) & 7)


def swz_v(row, key):
    return 4 * (key & 3) if row == 256 else 4 * ((key >> 1) & 1)


def dma_contents(row, keys, swz):
    """(key, physical chunk) -> (key, logical chunk) after the DMA of a tile
    of `keys` rows, as the kernels' per-lane DMA constants place it."""
    tb = keys * row
    ninst = tb // 1024
    per_wave = max(1, ninst // WAVES)
    held = {}
    writes = set()
    for wave in range(min(WAVES, ninst)):
        for q in range(per_wave):
            n = wave * per_wave + q
            for lane in range(64):
                byte = n * 1024 + 16 * lane            # LDS destination of this lane
                src = (wave * per_wave + q) * 1024 + 16 * lane
                key, pc = src // row, (src % row) // 16
                assert byte // row == key and (byte % row) // 16 == pc
                logical = pc ^ swz(row, key)
                held[(key, pc)] = (key, logical)
                writes.add(byte)
    assert len(writes) * 16 == tb, "the DMA must cover the tile exactly once"
    return held


def banks_of(addr, nbytes):
    return {((addr + b) // 4) % BANKS for b in range(0, nbytes, 4)}


def assert_conflict_free(addrs, nbytes, per_cycle):
    for c0 in range(0, len(addrs), per_cycle):
        used = set()
        for a in addrs[c0:c0 + per_cycle]:
            bk = banks_of(a, nbytes)
            assert not (used & bk), f"bank conflict among lanes {c0}..{c0 + per_cycle - 1}"
            used |= bk


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("keys", [64, 32])     # wide kernel tile, narrow kernel wave tile
def test_k_operand_reads(d, keys):
    row = 2 * d
    held = dma_contents(row, keys, swz_k)
    for kb in range(keys // 32):
        for ks in range(d // 16):
            addrs = []
            for lane in range(64):
                i, h = lane & 31, lane >> 5
                addr = i * row + 16 * ((2 * ks + h) ^ swz_k(row, i)) + kb * 32 * row
                key, pc = addr // row, (addr % row) // 16
                assert held[(key, pc)] == (32 * kb + i, 2 * ks + h), (kb, ks, lane)
                addrs.append(addr)
            assert_conflict_free(addrs, 16, 16)


def tr16_b64(words):
    """ds_read_b64_tr_b16 on one group of 16 lanes: `words[j]` are the four
    16-bit values lane j points at; lane j receives element j % 4 of lanes
    j // 4, 4 + j // 4, 8 + j // 4, 12 + j // 4 (a 4 x 16 block read row by
    row, handed out column by column)."""
    return [[words[4 * k + (j >> 2)][j & 3] for k in range(4)] for j in range(16)]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("keys", [64, 32])
def test_v_operand_reads(d, keys):
    row = 2 * d
    held = dma_contents(row, keys, swz_v)

    def element(addr):
        key, pc = addr // row, (addr % row) // 16
        k2, lc = held[(key, pc)]
        assert k2 == key
        return [(key, 8 * lc + (addr % 16) // 2 + e) for e in range(4)]   # (key, d) of 4 bf16 values

    for n in range(keys // 16):               # 16-key chunk of the tile
        for db in range(d // 32):             # 32-wide block of d
            got = [[] for _ in range(64)]
            for off in (0, 8 * row):          # keys + 0..3, then + 8..11
                addrs = []
                for g in range(4):
                    words = []
                    for j in range(16):
                        half, hh = g & 1, g >> 1
                        key0 = 4 * hh + (j >> 2)
                        addr = (key0 * row + 16 * ((4 * db + 2 * half + ((j >> 1) & 1)) ^ swz_v(row, key0))
                                + 8 * (j & 1) + 16 * n * row + off)
                        addrs.append(addr)
                        words.append(element(addr))
                    for j, vals in enumerate(tr16_b64(words)):
                        got[16 * g + j] += vals
                assert_conflict_free(addrs, 8, 32)
            for lane in range(64):
                i, h = lane & 31, lane >> 5
                # the P^T operand's key order for chunk n: slot e is key
                # 16 n + 8 (e // 4) + 4 h + e % 4 (the S^T accumulator layout)
                want = [(16 * n + 8 * (e >> 2) + 4 * h + (e & 3), 32 * db + i) for e in range(8)]
                assert got[lane] == want, (n, db, lane, got[lane], want)


def test_a_plausible_wrong_swizzle_is_caught():
    """The model is not vacuous: a V swizzle made for 32 banks (key & 1
    only) conflicts on 64 banks, and dropping the K swizzle conflicts too."""
    row = 256
    addrs = [(lane & 31) * row + 16 * ((2 * 0 + (lane >> 5)) ^ 0) for lane in range(64)]
    with pytest.raises(AssertionError):
        assert_conflict_free(addrs, 16, 16)
    addrs = []
    for j in range(32):
        key0 = j >> 2
        addrs.append(key0 * row + 16 * (((j >> 1) & 1) ^ (4 * (key0 & 1))) + 8 * (j & 1))
    with pytest.raises(AssertionError):
        assert_conflict_free(addrs, 8, 32)
