"""The direct K/V tile loads fill every LDS slot once, from the right bytes (CPU only).

Replays, for every wave, load and lane of a tile, the formulas the attention
kernels use to fetch K and V tiles by direct loads (global memory to LDS):

  * the lane offsets are computed once per pattern (koff[n % KPAT],
    voff[n % VPAT]) and reused for every load n of that pattern;
  * the rest of load n's source offset is a scalar offset, and at head dim
    512 (no ring or bias) also the load's immediate offset: the wave's loads
    fill contiguous 1 KiB blocks, four to one M0 value, load k of a group
    taking immediate 1024 k, which moves its LDS destination (M0 + immediate
    + 16 lane) and its source together;
  * the buffer descriptor of tile t starts at key row t BN and ends at key
    kL, and the range check covers vector + scalar + immediate offset.

Checks that every 16-byte LDS slot of the tile is written exactly once, with
the 16 source bytes of the key row and chunk the swizzled layout puts there
(chunk c of key row r at chunk position c ^ (r % 16) for K and
c ^ ((r % (VSW + 1)) * 4) for V), that rows at or past kL fall outside the
range (they read zeros), and that every immediate fits the 12-bit field.
The geometry restates the kernels': 4 waves, 64-key tiles of rows padded to
lds_row elements (32-key tiles of 512 at head dim 512), 1 KiB per load.
"""

import pytest

NW = 4
PAST_RANGE = 0x40000000


def lds_row(dk, dv):
    return 128 if max(dk, dv) <= 128 else 256 if max(dk, dv) <= 256 else 512


def replay(D, is_v, kL_in_tile, grp, mistake=None):
    LD = lds_row(D, D)
    BN = 32 if D == 512 else 64
    ROWCH = LD // 8
    TILE_BYTES = BN * LD * 2
    LOADS = TILE_BYTES // 1024 // NW
    RPB = 1024 // (2 * LD)
    VSW = 7 if ROWCH >= 32 else 3
    row_bytes = 2 * D
    if grp:
        KPAT = min(16 // RPB, LOADS)
        VPAT = min((VSW + 1) // RPB, LOADS)
    else:
        KPAT = max(16 // (NW * RPB), 1)
        VPAT = max((VSW + 1) // (NW * RPB), 1)
    assert LOADS % KPAT == 0 and LOADS % VPAT == 0
    if mistake == "pattern":  # lane offsets reused too early
        KPAT, VPAT = max(KPAT // 2, 1), max(VPAT // 2, 1)

    def blk(wave, n):
        return LOADS * wave + n if grp else wave + NW * n

    def swz_chunk(r, pch):
        return pch ^ ((r & VSW) << 2) if is_v else pch ^ (r & 15)

    def lane_off(wave, lane, n):
        r = blk(wave, n) * RPB + lane // ROWCH
        c = swz_chunk(r, lane % ROWCH)
        rn = n * RPB if grp else n * NW * RPB
        return (r - rn) * row_bytes + 16 * c if 16 * c < row_bytes else PAST_RANGE

    rng_bytes = min(kL_in_tile, BN) * row_bytes
    written = {}
    for wave in range(NW):
        pat = [[lane_off(wave, lane, i) for lane in range(64)] for i in range(VPAT if is_v else KPAT)]
        for n in range(LOADS):
            if grp:
                so, imm = (n & ~3) * 1024, (n & 3) * 1024
                if mistake == "scalar":  # the scalar offset not at the group's first block
                    so = n * 1024
                assert imm < 4096
                m0 = (LOADS * wave + (n & ~3)) * 1024
            else:
                so, imm = n * NW * RPB * row_bytes, 0
                m0 = blk(wave, n) * 1024
            for lane in range(64):
                vo = pat[n % len(pat)][lane]
                src = vo + so + imm
                dst = m0 + imm + 16 * lane
                assert 0 <= dst < TILE_BYTES
                assert dst not in written, (wave, n, lane)
                written[dst] = src if src < rng_bytes else None  # out of range: zeros
    assert len(written) == TILE_BYTES // 16
    # every slot holds what the swizzled layout puts there
    for dst, src in written.items():
        r, pch = dst // (2 * LD), (dst % (2 * LD)) // 16
        c = swz_chunk(r, pch)
        want = r * row_bytes + 16 * c
        if 16 * c >= row_bytes or r >= kL_in_tile:
            assert src is None, (dst, src)
        else:
            assert src == want, (dst, src, want)


@pytest.mark.parametrize("D,grp", [(512, True), (512, False), (256, False), (192, False), (128, False), (80, False), (64, False)])
@pytest.mark.parametrize("is_v", [False, True])
@pytest.mark.parametrize("kL_in_tile", [1, 7, 31, 32, 33, 64, 1000])
def test_tile_loads_fill_every_slot_once_from_its_bytes(D, grp, is_v, kL_in_tile):
    replay(D, is_v, kL_in_tile, grp)


@pytest.mark.parametrize("mistake", ["pattern", "scalar"])
def test_planted_mistakes_are_caught(mistake):
    """The replay is not vacuous: lane offsets reused every half pattern, or a
    scalar offset that also holds the immediate's block, fail the check."""
    with pytest.raises(AssertionError):
        replay(512, False, 32, True, mistake)
