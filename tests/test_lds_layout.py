"""The attention kernel's LDS layout, modelled on the CPU (host logic; no GPU).

The kernel copies each 128 x 256-byte K and V tile into LDS with an XOR swizzle of the
16-byte chunks of each row (csrc/common.h, row_swz) and reads the MFMA operands from it:
K rows with 16-byte reads, and, for a tile-major or raster V, the V^T operand of P V with
ds_read_b64_tr_b16, whose lane rule (within each 16-lane group, lane m receives element
m % 4 of what lane 4 r + m / 4 read, for r = 0..3) was established on the GPU with an
in-bounds probe.  This model replays the copy and both reads with the kernel's address
formulas and checks that
  - every lane's operand holds exactly the elements the MFMA expects (K[row][16 s + 8 hi ..],
    and V[key][32 db + lane % 32] for the keys 16 s + 4 hi + {0..3}, 16 s + 8 + 4 hi + {0..3}
    that the probabilities in k-slots 0-7 of the lane's P fragment belong to);
  - no read pass has two lanes on one bank, with 32 or with 64 four-byte banks (a pass
    being as many lanes as fill the banks once: 8 or 16 for 16-byte reads, 16 or 32 for
    8-byte reads);
  - the swizzle is a permutation of the 16 slots over any 16 aligned rows.
The swizzle table is read from csrc/common.h, so a change there is checked here."""
import os
import re

import numpy as np
import pytest

from conftest import ROOT

COMMON_H = os.path.join(ROOT, "video_dit_block_head_amd", "csrc", "common.h")


def quad_table():
    """g of SWZ_QUAD, swz(r) = g(r % 4) ^ ((r / 4) % 4), from the nibble constant in row_swz."""
    text = open(COMMON_H).read()
    m = re.search(r"\(\(\s*(0x[0-9A-Fa-f]+)\s*>>\s*\(4 \* \(r & 3\)\)\)\s*&\s*15\)\s*\^\s*\(\(r >> 2\) & 3\)", text)
    assert m, "row_swz's quad swizzle not found in csrc/common.h"
    c = int(m.group(1), 16)
    return [(c >> (4 * i)) & 15 for i in range(4)]


def swizzles():
    g = quad_table()
    return {"row": lambda r: r & 15, "quad": lambda r: g[r & 3] ^ ((r >> 2) & 3)}


def copy_tile(tile, swz):
    """The direct-to-LDS copy: wave w, instruction e, lane l -> tile row r = 32 w + 4 e + l / 16,
    LDS slot l % 16 of that row, source chunk slot ^ swz(r).  Returns the LDS image (bf16 units)."""
    lds = np.full(128 * 128, -1, dtype=np.int64)
    for w in range(4):
        for e in range(8):
            for lane in range(64):
                r = 32 * w + 4 * e + lane // 16
                chunk = (lane % 16) ^ swz(r)
                dst = ((32 * w + 4 * e) * 256 + 16 * lane) // 2
                lds[dst:dst + 8] = tile[r, 8 * chunk:8 * chunk + 8]
    assert (lds >= 0).all()
    return lds


def conflict_free(addrs, nbytes):
    """Bank check of one read instruction (byte address per lane, nbytes per lane): the lanes
    are serviced in passes of as many lanes as fill the banks once (32 or 64 four-byte
    banks), and no pass may touch a bank twice."""
    for banks in (32, 64):
        group = banks * 4 // nbytes
        for g0 in range(0, 64, group):
            hit = [((a // 4) + x) % banks for a in addrs[g0:g0 + group] for x in range(nbytes // 4)]
            if len(set(hit)) != len(hit):
                return False
    return True


@pytest.fixture(scope="module")
def tile():
    return np.arange(128 * 128, dtype=np.int64).reshape(128, 128)   # element (row, col) = 128 row + col


@pytest.mark.parametrize("name", ["row", "quad"])
def test_swizzle_is_a_permutation_and_k_reads_are_exact(tile, name):
    swz = swizzles()[name]
    for base in range(0, 128, 16):
        assert sorted(swz(base + i) for i in range(16)) == list(range(16))
    lds = copy_tile(tile, swz)
    for kb in range(4):
        for s in range(8):
            addrs = []
            for lane in range(64):
                lr, hi = lane % 32, lane // 32
                row = 32 * kb + lr
                a = row * 256 + 16 * ((2 * s + hi) ^ swz(lr))     # the kernel's K operand read
                addrs.append(a)
                assert list(lds[a // 2:a // 2 + 8]) == list(tile[row, 16 * s + 8 * hi:16 * s + 8 * hi + 8])
            assert conflict_free(addrs, 16), (name, kb, s)


def test_transposed_v_reads_give_the_mfma_operand(tile):
    swz = swizzles()["quad"]
    lds = copy_tile(tile, swz)

    def tr_read(addrs):
        got = [lds[a // 2:a // 2 + 4] for a in addrs]
        return [[got[16 * (lane // 16) + 4 * r + (lane % 16) // 4][lane % 4] for r in range(4)]
                for lane in range(64)]

    for s in range(8):
        for db in range(4):
            halves = []
            for p in range(2):
                addrs = []
                for lane in range(64):
                    hi, i16 = lane // 32, lane % 16
                    rq = i16 // 4
                    cb = 2 * ((lane // 16) % 2) + (i16 % 4) // 2
                    slot = (4 * db + cb) ^ swz(8 * p + 4 * hi + rq)
                    a = (4 * hi + rq) * 256 + 16 * slot + 8 * (i16 % 2) + 4096 * s + 2048 * p
                    assert a % 8 == 0 and 0 <= a <= 32768 - 8
                    addrs.append(a)
                assert conflict_free(addrs, 8), (s, db, p)
                halves.append(tr_read(addrs))
            for lane in range(64):
                lr, hi = lane % 32, lane // 32
                keys = [16 * s + 8 * (e // 4) + 4 * hi + e % 4 for e in range(8)]
                assert halves[0][lane] + halves[1][lane] == [tile[k, 32 * db + lr] for k in keys], (s, db, lane)


def test_row_swizzle_would_conflict_on_transposed_reads(tile):
    """The plain r & 15 swizzle serves the K reads but not the transposed V reads: four
    consecutive rows then share their slots, which is why V tiles read that way (and K
    with them) use the quad swizzle."""
    swz = swizzles()["row"]
    addrs = []
    for lane in range(64):
        hi, i16 = lane // 32, lane % 16
        rq = i16 // 4
        cb = 2 * ((lane // 16) % 2) + (i16 % 4) // 2
        addrs.append((4 * hi + rq) * 256 + 16 * (cb ^ swz(4 * hi + rq)) + 8 * (i16 % 2))
    assert not conflict_free(addrs, 8)
