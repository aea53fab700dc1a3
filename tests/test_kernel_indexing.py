"""Host emulation of the kernel's index arithmetic (no GPU).

Restates, in numpy, the address formulas of
attention_forward_fa2_amd/csrc/fa2_fwd_kernel.hip for the tile shapes the
library uses and checks, for many tensor shapes, that
  * the workgroup -> (head, query tile) mapping is a bijection,
  * every global load (Q rows, K/V tiles, clamped ragged tiles) and every store
    (O, LSE) stays inside its tensor,
  * every LDS destination and LDS read stays inside the ring,
  * the hoisted per-lane LDS read offsets equal the per-row formulas,
  * the XOR swizzles put each ds_read_b128 quarter-wave (K) and each
    transposing-read half-wave (V) on distinct 16-byte bank groups of a
    256-byte window,
  * the transposing reads deliver V[32kc + 4g + e][16db + lane%16] in element e,
    in the key order of the S^T accumulator (the P handoff).
If the kernel's formulas change, this file must change with them."""
import numpy as np
import pytest


def swz_k(D, r):
    return ((r >> 1) & 7) if D == 64 else (r & 15)


def swz_v(D, r):
    return (((r >> 1) & 3) << 1) if D == 64 else ((r & 7) << 1)


# D -> (QB, NW, BN, SUB) of the library's tiles (SUB compute tiles per LDS stage)
SHAPES = {64: (2, 8, 64, 2), 128: (2, 8, 64, 2)}
VARIANTS = [(2, 8, 64, 1), (2, 8, 64, 2), (2, 4, 64, 1), (2, 4, 64, 2), (4, 4, 64, 1)]


def block_map(BH, nqt, causal):
    nb = BH * nqt
    bid = np.arange(nb)
    xcd, slot = bid & 7, bid >> 3
    if causal and BH % 8 == 0:
        hx = BH >> 3
        return xcd + 8 * (slot % hx), nqt - 1 - slot // hx
    per, rem = nb >> 3, nb & 7
    logical = xcd * per + np.minimum(xcd, rem) + slot
    if causal:
        return logical % BH, nqt - 1 - logical // BH
    return logical // nqt, logical % nqt


@pytest.mark.parametrize("BH", list(range(1, 41)) + [96, 192, 256])
@pytest.mark.parametrize("nqt", [1, 2, 3, 16, 33])
@pytest.mark.parametrize("causal", [False, True])
def test_block_mapping_is_a_bijection(BH, nqt, causal):
    bh, qt = block_map(BH, nqt, causal)
    assert bh.min() >= 0 and bh.max() < BH and qt.min() >= 0 and qt.max() < nqt
    assert len(set(zip(bh.tolist(), qt.tolist()))) == BH * nqt


def emulate(B, H, S, D, causal, shape=None):
    QB, NW, BN, SUB = shape or SHAPES[D]
    QW, BM = 16 * QB, 16 * QB * NW
    CPR, TILE, DB, NKC, NKB, DK = D // 8, BN * D, D // 16, BN // 32, BN // 16, D // 32
    KB, LTILE = SUB * BN, SUB * BN * D
    LOADS = LTILE // 8 // 64 // NW
    RPL = NW * 64 // CPR
    assert RPL % 16 == 0
    lane = np.arange(64)
    l16, g = lane & 15, lane >> 4
    nqt = -(-S // BM)
    bh, qt = block_map(B * H, nqt, causal)
    total = B * H * S * D
    for wave in range(NW):
        qw0 = qt * BM + wave * QW
        # Q loads (rows clamped to S-1)
        for qb in range(QB):
            row = np.minimum(qw0[:, None] + 16 * qb + l16[None, :], S - 1)
            for kk in range(DK):
                off = bh[:, None] * S * D + row * D + 32 * kk + 8 * g[None, :]
                assert off.min() >= 0 and (off + 8).max() <= total
        # K/V direct-to-LDS loads: the kernel keeps one lane offset (row0, pc0)
        # per tensor and steps the scalar base by RPL rows per load
        row0, pc0 = (wave * 64 + lane) // CPR, lane % CPR
        for i in range(LOADS):
            c = (i * NW + wave) * 64 + lane
            r, pc = c // CPR, c % CPR
            assert np.array_equal(r, row0 + i * RPL) and np.array_equal(pc, pc0)
            dst = 2 * (i * NW + wave) * 512 + 16 * lane
            assert dst.min() >= 0 and (dst + 16).max() <= 2 * LTILE
            for sw in (swz_k, swz_v):
                generic = r * D + 8 * (pc ^ sw(D, r))
                lane_off = row0 * D + 8 * (pc0 ^ sw(D, row0))
                assert np.array_equal(generic, lane_off + i * RPL * D)
                for t in range(-(-S // KB)):
                    k0 = t * KB
                    if k0 + KB <= S:
                        el = (k0 + i * RPL) * D + lane_off
                    else:
                        el = (np.minimum(k0 + r, S - 1) - row0) * D + lane_off
                        ok = k0 + r < S
                        assert np.array_equal(el[ok], (k0 * D + generic)[ok])
                    assert el.min() >= 0 and (el + 8).max() <= S * D
        # O and LSE stores
        for qb in range(QB):
            row = qw0[:, None] + 16 * qb + l16[None, :]
            ok = row < S
            if not ok.any():
                continue
            for db in range(DB):
                off = bh[:, None] * S * D + row * D + 16 * db + 4 * g[None, :]
                assert off[ok].min() >= 0 and (off[ok] + 4).max() <= total
            lo = bh[:, None] * S + row
            assert lo[ok].min() >= 0 and lo[ok].max() < B * H * S


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 2, 15, 16, 17, 63, 64, 65, 127, 129, 255, 257, 320, 513, 1000, 4096])
@pytest.mark.parametrize("causal", [False, True])
def test_global_accesses_in_bounds(D, S, causal):
    emulate(1, 3, S, D, causal)
    emulate(2, 4, S, D, causal)


@pytest.mark.parametrize("shape", VARIANTS, ids=[f"QB{a}NW{b}BN{c}SUB{d}" for a, b, c, d in VARIANTS])
@pytest.mark.parametrize("D", [64, 128])
def test_global_accesses_in_bounds_other_tilings(shape, D):
    for S in (1, 63, 65, 129, 257, 1000):
        for causal in (False, True):
            emulate(2, 3, S, D, causal, shape)


@pytest.mark.parametrize("D", [64, 128])
def test_lds_reads_and_bank_groups(D):
    QB, NW, BN, SUB = SHAPES[D]
    TILE, DB, NKC, NKB, DK = BN * D, D // 16, BN // 32, BN // 16, D // 32
    lane = np.arange(64)
    l16, g = lane & 15, lane >> 4
    for kk in range(DK):
        hoisted = 2 * (l16 * D + 8 * ((4 * kk + g) ^ swz_k(D, l16)))
        for kb in range(NKB):
            r = 16 * kb + l16
            direct = 2 * (r * D + 8 * ((4 * kk + g) ^ swz_k(D, r)))
            assert np.array_equal(hoisted + kb * 16 * D * 2, direct)
            assert direct.min() >= 0 and (direct + 16).max() <= 2 * TILE
            for quarter in range(4):  # ds_read_b128: 16 lanes per 256-byte window
                groups = (direct[16 * quarter:16 * quarter + 16] // 16) % 16
                assert len(set(groups.tolist())) == 16
    r0 = 4 * g + (l16 >> 2)
    for db in range(DB):
        lc = 2 * db + ((l16 & 3) >> 1)
        hoisted = 2 * (r0 * D + 8 * (lc ^ swz_v(D, r0)) + 4 * (l16 & 1))
        for kc in range(NKC):
            for half in (0, 1):
                r = 32 * kc + 16 * half + r0
                direct = 2 * (r * D + 8 * (lc ^ swz_v(D, r)) + 4 * (l16 & 1))
                assert np.array_equal(hoisted + kc * 32 * D * 2 + half * 16 * D * 2, direct)
                assert direct.min() >= 0 and (direct + 8).max() <= 2 * TILE
                for hw in range(2):  # 8-byte reads: 32 lanes per 256-byte window
                    groups = (direct[32 * hw:32 * hw + 32] // 16) % 16
                    assert len(set(groups.tolist())) == 16


def tr16(addrs_elems, lds):
    """ds_read_b64_tr_b16 as measured on the device: within each 16-lane group,
    lane i receives element i%4 of the 4 values loaded by lane i//4 + 4e."""
    loaded = np.stack([lds[a:a + 4] for a in addrs_elems])  # [64, 4]
    out = np.empty((64, 4), dtype=lds.dtype)
    for grp in range(4):
        for i in range(16):
            for e in range(4):
                out[16 * grp + i, e] = loaded[16 * grp + i // 4 + 4 * e, i % 4]
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_reads_match_the_score_layout(D):
    """The V^T operand must list, for lane (d = 16db + lane%16, g = lane/16),
    the keys 32kc + 4g + e (first read) and 32kc + 16 + 4g + e (second read):
    the keys the S^T accumulator of that lane holds (16-key blocks 2kc, 2kc+1)."""
    BN = SHAPES[D][2] * 2  # two compute tiles: a sub-tile starts at a multiple of BN rows
    # LDS tile as the DMA writes it: row r, physical chunk pc holds logical chunk pc ^ swz_v(r)
    key_of = np.zeros(BN * D, dtype=np.int64)
    col_of = np.zeros(BN * D, dtype=np.int64)
    for r in range(BN):
        for pc in range(D // 8):
            lc = pc ^ swz_v(D, r)
            for x in range(8):
                key_of[r * D + 8 * pc + x] = r
                col_of[r * D + 8 * pc + x] = 8 * lc + x
    lane = np.arange(64)
    l16, g = lane & 15, lane >> 4
    r0 = 4 * g + (l16 >> 2)
    for db in range(D // 16):
        lc = 2 * db + ((l16 & 3) >> 1)
        base = r0 * D + 8 * (lc ^ swz_v(D, r0)) + 4 * (l16 & 1)
        for kc in range(BN // 32):  # key chunks of both sub-tiles
            for half in (0, 1):
                a = base + kc * 32 * D + half * 16 * D
                keys, cols = tr16(a, key_of), tr16(a, col_of)
                for e in range(4):
                    assert np.array_equal(keys[:, e], 32 * kc + 16 * half + 4 * g + e)
                    assert np.array_equal(cols[:, e], 16 * db + l16)
