"""The bias loads of the attention kernels read no byte outside the bias (CPU only).

Replays, for every workgroup, tile, wave, load and lane of a launch, the
formulas the bias instances use to fetch their tiles: the lane's byte offset
(its packed row's query head and position through the bias strides, plus its
8-key chunk, or an offset past the range for rows beyond the workgroup), the
buffer descriptor of a tile (base at key t * BN of batch b's bias, range to
the end of the batch's extent) and its per-4-byte-word range check, then the
one element written in afterwards when kL is odd.  Checks that

  * every word the hardware would fetch lies inside [0, extent) elements of
    batch b's bias, so a bias may end on any page boundary, and
  * every key below kL of every packed row a workgroup holds lands in the
    tile with the bias's own value (the words out of range read as zero;
    only keys at or past kL may keep that zero).

The geometry constants restate the kernels': 4 waves, 128 packed rows and
64-key tiles (64 rows and 32-key tiles at head dim 512), 8 keys (16 bytes)
per lane and load, chunk c of tile row r stored at chunk position
c ^ (r % chunks_per_row).
"""

import numpy as np
import pytest

NW = 4


def geometry(D):
    BM, BN = (64, 32) if D == 512 else (128, 64)
    BCPR = BN * 2 // 16
    BRPB = 64 // BCPR
    BLOADS = BM * BN * 2 // 1024 // NW
    return BM, BN, BCPR, BRPB, BLOADS


def replay(B, Hq, Hkv, qL, kL, D, sb, sh, sq, causal, q_offset, nsplit=1, split_len=None, slack=0):
    """Returns (end of the elements fetched, relative to batch b's bias start,
    the extent, the number of keys below kL that hold a wrong value)."""
    BM, BN, BCPR, BRPB, BLOADS = geometry(D)
    G = Hq // Hkv
    rows = G * qL
    mblocks = -(-rows // BM)
    split_len = split_len or kL
    extent = (Hq - 1) * sh + (qL - 1) * sq + kL
    last_row = extent - kL
    c_last = ((kL - 1) % BN) // 8
    t_bend = (kL - 1) // BN
    rng = np.random.default_rng(B * 7 + kL)
    bias = rng.integers(1, 60000, size=(B - 1) * sb + extent, dtype=np.int64)  # nonzero values
    worst, wrong = -1, 0
    wave = np.repeat(np.arange(NW), 64)[:, None]        # [256, 1]
    lane = np.tile(np.arange(64), NW)[:, None]
    n = np.arange(BLOADS)[None, :]                      # [1, BLOADS]
    r = (wave + NW * n) * BRPB + lane // BCPR           # tile row of each (thread, load)
    pos_lds = lane % BCPR
    c = pos_lds ^ (r & (BCPR - 1))                      # the logical chunk it fetches
    for b in range(B):
        for hkv in range(Hkv):
            for mb in range(mblocks):
                row0 = mb * BM
                rows_end = min(rows, row0 + BM)
                prow = row0 + r
                valid = prow < rows_end
                pq, ph = prow // G, hkv * G + prow % G
                start = ph * sh + pq * sq
                boff = np.where(valid, (start + 8 * c) * 2, 0xFFFFFFF0)
                bp_lo = q_offset + row0 // G
                bp_hi = q_offset + (rows_end - 1) // G
                for s in range(nsplit):
                    kbeg, kend = 0, kL
                    if causal:
                        kend = min(kend, bp_hi + 1)
                    kbeg, kend = max(kbeg, s * split_len), min(kend, (s + 1) * split_len)
                    if kbeg >= kend:
                        continue
                    t_first, t_last = kbeg // BN, (kend - 1) // BN
                    patch = (kL % 2 == 1) & valid & (start == last_row) & (c == c_last) & (t_last == t_bend)
                    for t in range(t_first, t_last + 1):
                        ts = t * BN
                        rng_bytes = (extent - ts) * 2 + slack
                        tile = np.zeros((BM, BN), dtype=np.int64)
                        for w in range(4):  # the four 4-byte words of a lane's 16 bytes
                            off = boff + 4 * w
                            inr = off + 4 <= rng_bytes
                            el0 = ts + off // 2              # element index of the word's first half
                            if inr.any():
                                worst = max(worst, int(el0[inr].max()) + 2)  # exclusive end
                                assert int(el0[inr].min()) >= 0
                            for half in range(2):
                                el = el0 + half
                                val = np.where(inr, bias[np.clip(b * sb + el, 0, bias.size - 1)], 0)
                                key = 8 * c + 2 * w + half
                                m = valid
                                tile[r[m], key[m]] = val[m]
                        if t == t_bend:  # the element the range check zeroed
                            e = (kL - 1) % 8
                            tile[r[patch], (8 * c + e)[patch]] = bias[b * sb + last_row + kL - 1]
                        # every key below kL of every held row must hold its bias value
                        rr = np.arange(rows_end - row0)
                        pr = row0 + rr
                        st = (hkv * G + pr % G) * sh + (pr // G) * sq
                        keys = ts + np.arange(BN)
                        ok = keys < kL
                        want = bias[b * sb + st[:, None] + np.minimum(keys, kL - 1)[None, :]]
                        got = tile[rr][:, :BN]
                        wrong += int(((got != want) & ok[None, :]).sum())
    return worst, extent, wrong


CASES = [
    # B, Hq, Hkv, qL, kL, D, sb, sh, sq, causal, q_offset
    (1, 16, 8, 128, 4097, 256, 0, 128 * 4097, 4097, True, 4097 - 128),   # contiguous, odd kL
    (2, 12, 3, 3, 3, 256, 0, 9, 3, True, 0),                             # per-head bias shared by the batch
    (1, 2, 1, 5, 333, 256, 0, 0, 0, True, 328),                          # one row shared by all
    (2, 4, 2, 33, 333, 256, 4 * 33 * 333, 33 * 333, 333, True, 300),     # full bias, odd row starts
    (1, 4, 2, 40, 335, 256, 0, 0, 336, False, 0),                        # row stride kL + 1 (a view)
    (1, 4, 1, 70, 171, 512, 0, 70 * 171, 171, True, 101),                # head dim 512 tiles
    (2, 2, 1, 31, 97, 512, 2 * 31 * 98, 31 * 98, 98, False, 0),          # head dim 512, even stride
    (1, 4, 2, 50, 200, 128, 0, 50 * 201, 201, True, 150),                # odd row stride, even kL
    (1, 8, 2, 20, 1001, 64, 0, 20 * 1001, 1001, True, 981),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}q{c[3]}k{c[4]}D{c[5]}s{c[7]}_{c[8]}" for c in CASES])
def test_bias_fetches_stay_inside_the_extent(case):
    B, Hq, Hkv, qL, kL, D, sb, sh, sq, causal, q_offset = case
    worst, extent, wrong = replay(B, Hq, Hkv, qL, kL, D, sb, sh, sq, causal, q_offset)
    assert worst <= extent, (worst, extent)
    assert wrong == 0, wrong


def test_bias_fetches_stay_inside_the_extent_with_key_splits():
    # a split call: each split's workgroups fetch only their own tiles
    worst, extent, wrong = replay(1, 2, 1, 300, 9001, 256, 0, 300 * 9001, 9001, True, 8701,
                                  nsplit=3, split_len=3072)
    assert worst <= extent and wrong == 0, (worst, extent, wrong)


def test_the_replay_catches_a_range_two_bytes_long():
    # the range of the earlier kernels (extent + 2 bytes): the replay must see
    # the word past the extent
    worst, extent, _ = replay(1, 16, 8, 128, 4097, 256, 0, 128 * 4097, 4097, True, 4097 - 128, slack=2)
    assert worst == extent + 1
