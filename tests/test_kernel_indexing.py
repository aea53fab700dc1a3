"""Host emulation of the kernel's index arithmetic (no GPU).

Restates, in numpy, the address formulas of
attention_forward_fa2_amd/csrc/fa2_fwd_kernel.hip for the tile shapes the
library uses and checks, for many tensor shapes, that
  * the workgroup -> (head, query tile) mapping is a bijection, also when
    query heads share K/V heads (GQA/MQA),
  * every global load (Q rows, K/V tiles, clamped ragged tiles) and every store
    (O, LSE) stays inside its tensor and inside its own sequence, for the
    dense [B,H,S,D] layout and for packed sequences [total,H,D] (including
    malformed sequence tables, which the kernel clamps),
  * the K/V stages a workgroup scans and the compute tiles each wave keeps
    cover every admissible key of its rows (causal and local windows), and a
    tile the kernel does not mask holds only admissible keys,
  * the dropout counter of each probability register names that register's key,
  * every LDS destination and LDS read stays inside the ring,
  * the per-lane LDS read offsets (one base per tensor, XORed with the k-step
    or column block) equal the per-row formulas,
  * the XOR swizzles put each ds_read_b128 quarter-wave (K) and each
    transposing-read half-wave (V) on distinct 16-byte bank groups of a
    256-byte window,
  * the transposing reads deliver V[32kc + 4g + e][16db + lane%16] in element e,
    in the key order of the S^T accumulator (the P handoff).
The workgroup mapping, the swizzles, the per-lane K/V load offsets and the LDS
read bases restated here are also compared with the kernel's own code: they
live in attention_forward_fa2_amd/csrc/fa2_index.h, which a host-only probe
library (tests/index_probe) compiles for the CPU. The other formulas (the loop
bounds, masks, stores) are restated only; if they change in the kernel, this
file must change with them."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def swz_k(D, r):
    return ((r >> 1) & 7) if D == 64 else (r & 15)


def swz_v(D, r):
    return (((r >> 1) & 3) << 1) if D == 64 else ((r & 7) << 1)


def lane_load_offsets(D, NW, kv_sr, wave, lane):
    """A lane's first stage row and its K and V source offsets (bytes)."""
    CPR = D // 8
    row0, pc0 = (wave * 64 + lane) // CPR, lane % CPR
    return (row0, 2 * (row0 * kv_sr + 8 * (pc0 ^ swz_k(D, row0))),
            2 * (row0 * kv_sr + 8 * (pc0 ^ swz_v(D, row0))))


def lds_read_bases(D, lane):
    """The per-lane K and V LDS read bases (bytes) of the 16x16x32 path."""
    l16, g = lane & 15, lane >> 4
    rdK0 = 2 * (l16 * D + 8 * (g ^ swz_k(D, l16)))
    r0v = 4 * g + (l16 >> 2)
    rdV0 = 2 * (r0v * D + 8 * (((l16 & 3) >> 1) ^ swz_v(D, r0v)) + 4 * (l16 & 1))
    return rdK0, rdV0


# D -> (QB, NW, BN, SUB) of the library's tiles (SUB compute tiles per LDS stage)
SHAPES = {64: (2, 8, 64, 2), 128: (2, 8, 64, 2)}
VARIANTS = [(2, 8, 64, 1), (2, 8, 64, 2), (2, 4, 64, 1), (2, 4, 64, 2), (4, 4, 64, 1)]


def sequence_of_rank(lens, rho):
    """The kernel's ranking: the sequence whose count of sequences ranking
    before it (longer, or as long with a lower index) is rho."""
    n = len(lens)
    ranks = [sum((lens[i] > lens[j]) or (lens[i] == lens[j] and i < j) for i in range(n)) for j in range(n)]
    hits = [j for j in range(n) if ranks[j] == rho]
    assert len(hits) == 1
    return hits[0]


def block_map_packed(BH, nqt, causal, group=1, lens=None):
    """Packed sequences: (sequence, K/V head) unit u on XCD u mod 8, unit by
    unit; with lens given (at most 64 sequences) the units are numbered
    longest sequence first. Returns (bh, qt, valid) over the padded grid."""
    BHkv = BH // group
    nb = -(-BHkv // 8) * 8 * nqt * group
    bid = np.arange(nb)
    xcd, slot = bid & 7, bid >> 3
    per_unit = nqt * group
    kvu = xcd + 8 * (slot // per_unit)
    rem = slot % per_unit
    valid = kvu < BHkv
    if lens is not None:
        H_kv = BHkv // len(lens)
        order = [sequence_of_rank(lens, r) for r in range(len(lens))]
        kvu = np.where(valid, np.array(order + [0])[np.minimum(kvu // H_kv, len(lens))] * H_kv + kvu % H_kv, kvu)
    qt = rem // group
    if causal:
        qt = nqt - 1 - qt
    return kvu * group + rem % group, qt, valid


@pytest.mark.parametrize("BHkv", [1, 3, 8, 12, 24, 40])
@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("nqt", [1, 3, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_mapping(BHkv, group, nqt, causal):
    """Every (unit, query tile) exactly once among the valid workgroups, each
    K/V unit's workgroups on XCD unit mod 8."""
    BH = BHkv * group
    bh, qt, ok = block_map_packed(BH, nqt, causal, group)
    bh, qt = bh[ok], qt[ok]
    assert bh.min() >= 0 and bh.max() < BH and qt.min() >= 0 and qt.max() < nqt
    assert len(set(zip(bh.tolist(), qt.tolist()))) == BH * nqt == ok.sum()
    xcd = np.nonzero(ok)[0] & 7
    assert np.array_equal(xcd, (bh // group) % 8)


@pytest.mark.parametrize("nseq", [1, 2, 7, 24, 64])
@pytest.mark.parametrize("H_kv,group", [(1, 1), (2, 4), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_mapping_longest_first(nseq, H_kv, group, causal):
    """Longest-first packed order: still every (unit, query tile) exactly once
    among the valid workgroups and each K/V unit on one XCD; along the unit
    numbering the sequence lengths never increase; ties and empty sequences
    (a malformed table clamps to such lengths) keep it a bijection."""
    g = np.random.Generator(np.random.PCG64(nseq * 31 + H_kv))
    lens = [int(x) if g.random() > 0.2 else int(g.choice([0, 5])) for x in g.integers(0, 3000, size=nseq)]
    BH, nqt = nseq * H_kv * group, 3
    bh, qt, ok = block_map_packed(BH, nqt, causal, group, lens)
    bh, qt = bh[ok], qt[ok]
    assert len(set(zip(bh.tolist(), qt.tolist()))) == BH * nqt == ok.sum()
    kv = bh // group
    xcd = np.nonzero(ok)[0] & 7
    for u in range(nseq * H_kv):
        assert len(set(xcd[kv == u].tolist())) == 1
    order = [sequence_of_rank(lens, r) for r in range(nseq)]
    assert [lens[b] for b in order] == sorted(lens, reverse=True)


def block_map(BH, nqt, causal, group=1, serp=0):
    """serp: workgroups per serpentine band (the host passes the CUs per XCD
    when the grid is resident in one round), 0 for the heaviest-first walk."""
    nb = BH * nqt
    bid = np.arange(nb)
    xcd, slot = bid & 7, bid >> 3
    BHkv = BH // group
    if causal and BHkv % 8 == 0:
        per_tile = (BHkv >> 3) * group
        s = slot.copy()
        if serp:
            band = s // serp
            back = ((band & 1) == 1) & ((band + 1) * serp <= (nb >> 3))
            s = np.where(back, band * serp + (serp - 1 - s % serp), s)
        r = s % per_tile
        return (xcd + 8 * (r // group)) * group + r % group, nqt - 1 - s // per_tile
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


@pytest.mark.parametrize("BHkv,group", [(8, 1), (16, 1), (32, 1), (64, 1), (8, 4), (24, 2)])
@pytest.mark.parametrize("nqt", [1, 5, 8, 16, 32, 33, 64])
def test_serpentine_causal_mapping(BHkv, group, nqt):
    """One-round causal grids: with 32 workgroups per band the walk is still a
    bijection, keeps each K/V head on one XCD, and when slot s of an XCD lands
    on compute unit s mod 32 every compute unit of an XCD receives the same
    number of key tiles to scan, up to one band's spread (the last, partial
    band is not reversed)."""
    BH = BHkv * group
    bh, qt = block_map(BH, nqt, True, group, serp=32)
    assert bh.min() >= 0 and bh.max() < BH and qt.min() >= 0 and qt.max() < nqt
    assert len(set(zip(bh.tolist(), qt.tolist()))) == BH * nqt
    xcd = np.arange(BH * nqt) & 7
    kv = bh // group
    for h in range(BHkv):
        assert len(set(xcd[kv == h].tolist())) == 1
    slots = BH * nqt // 8
    if slots % 64 == 0:  # whole pairs of bands: every compute unit gets the same load
        for x in range(8):
            work = (qt + 1)[xcd == x]          # key tiles scanned, in slot order
            load = np.bincount(np.arange(slots) % 32, weights=work, minlength=32)
            assert load.max() == load.min()
    plain_bh, plain_qt = block_map(BH, nqt, True, group)
    if slots <= 32:  # a single band is never reversed
        assert np.array_equal(bh, plain_bh) and np.array_equal(qt, plain_qt)


@pytest.mark.parametrize("BHkv,group", [(8, 2), (8, 4), (16, 3), (24, 8), (32, 1), (4, 4), (12, 2), (1, 32)])
@pytest.mark.parametrize("nqt", [1, 5, 16])
def test_gqa_causal_mapping(BHkv, group, nqt):
    """Causal with GQA: a bijection, and when the K/V heads split evenly over
    the 8 XCDs every query head of one K/V head lands on one XCD."""
    BH = BHkv * group
    bh, qt = block_map(BH, nqt, True, group)
    assert bh.min() >= 0 and bh.max() < BH and qt.min() >= 0 and qt.max() < nqt
    assert len(set(zip(bh.tolist(), qt.tolist()))) == BH * nqt
    if BHkv % 8 == 0:
        xcd = np.arange(BH * nqt) & 7
        kv = bh // group
        for h in range(BHkv):
            assert len(set(xcd[kv == h].tolist())) == 1


def emulate(B, H, S, D, causal, shape=None, H_kv=None, cu=None, total=None, window=None):
    """Walk every workgroup and wave of one launch with the kernel's formulas.
    Dense: q/o [B,H,S,D], k/v [B,H_kv,S,D], lse [B,H,S]. Packed (cu given): B
    sequences, q/o [total,H,D], k/v [total,H_kv,D], lse [H,total], S = longest
    sequence. window = (wl, wr) as the host passes it (after clamping unbounded
    sides to S); causal = (S, 0) uses the causal kernel."""
    QB, NW, BN, SUB = shape or SHAPES[D]
    H_kv = H_kv or H
    group = H // H_kv
    QW, BM = 16 * QB, 16 * QB * NW
    CPR, DB, DK = D // 8, D // 16, D // 32
    KB, LTILE = SUB * BN, SUB * BN * D
    LOADS = LTILE // 8 // 64 // NW
    RPL = NW * 64 // CPR
    assert RPL % 16 == 0
    mode = "window" if window is not None else ("causal" if causal else "none")
    wl, wr = window if window is not None else (S, 0 if causal else S)
    if cu is None:
        q_sr, q_sh, q_sb = D, S * D, H * S * D
        kv_sr, kv_sh, kv_sb = D, S * D, H_kv * S * D
        l_sh, l_sb = S, H * S
        n_q, n_kv, n_l = B * H * S * D, B * H_kv * S * D, B * H * S
        rows_total = None
    else:
        q_sr, q_sh, q_sb = H * D, D, 0
        kv_sr, kv_sh, kv_sb = H_kv * D, D, 0
        l_sh, l_sb = total, 0
        n_q, n_kv, n_l = total * H * D, total * H_kv * D, H * total
    lane = np.arange(64)
    l16, g = lane & 15, lane >> 4
    nqt = -(-S // BM)
    if cu is None:
        bhs, qts = block_map(B * H, nqt, mode == "causal", group)
    else:
        # the kernel's clamped lengths, ranked longest first for up to 64 sequences
        lens = []
        for i in range(B):
            s0 = min(max(int(cu[i]), 0), total)
            lens.append(min(min(max(int(cu[i + 1]), s0), total) - s0, S))
        bhs, qts, valid = block_map_packed(B * H, nqt, mode == "causal", group, lens if B <= 64 else None)
        bhs, qts = bhs[valid], qts[valid]
        assert len(set(zip(bhs.tolist(), qts.tolist()))) == B * H * nqt
    for bh, qt in zip(bhs.tolist(), qts.tolist()):
        b, h = divmod(bh, H)
        hk = h // group
        start, ln = 0, S
        if cu is not None:
            s0 = min(max(cu[b], 0), total)
            s1 = min(max(cu[b + 1], s0), total)
            start, ln = s0, min(s1 - s0, S)
        q0 = qt * BM
        if q0 >= ln:
            continue
        qbase = b * q_sb + h * q_sh + start * q_sr
        kvbase = b * kv_sb + hk * kv_sh + start * kv_sr
        lbase = b * l_sb + h * l_sh + start
        q_last = min(q0 + BM, ln) - 1
        kbeg, kend = 0, ln
        if mode == "causal":
            kend = q_last + 1
        if mode == "window":
            kbeg, kend = max(0, q0 - wl), min(ln, q_last + wr + 1)
        t_begin, t_end = kbeg // KB, -(-kend // KB)
        for wave in range(NW):
            qw0 = q0 + wave * QW
            # Q loads (rows clamped to len-1, inside the sequence)
            for qb in range(QB):
                row = np.minimum(qw0 + 16 * qb + l16, ln - 1)
                for kk in range(DK):
                    off = qbase + row * q_sr + 32 * kk + 8 * g
                    assert off.min() >= 0 and (off + 8).max() <= n_q
                    assert (start + row).min() >= start and (start + row).max() < start + ln
            # K/V direct-to-LDS loads: one lane offset per tensor, scalar steps
            row0, offK, offV = lane_load_offsets(D, NW, kv_sr, wave, lane)
            pc0 = lane % CPR
            for i in range(LOADS):
                c = (i * NW + wave) * 64 + lane
                r, pc = c // CPR, c % CPR
                assert np.array_equal(r, row0 + i * RPL) and np.array_equal(pc, pc0)
                dst = 2 * (i * NW + wave) * 512 + 16 * lane
                assert dst.min() >= 0 and (dst + 16).max() <= 2 * LTILE
                for sw, off in ((swz_k, offK), (swz_v, offV)):
                    assert off.max() < 2 ** 32
                    lane_off = off // 2
                    for t in range(t_begin, t_end):
                        k0 = t * KB
                        if k0 + KB <= ln:
                            el = kvbase + (k0 + i * RPL) * kv_sr + lane_off
                            krow = k0 + r
                        else:
                            krow = np.minimum(k0 + r, ln - 1)
                            el = kvbase + (krow - row0) * kv_sr + lane_off
                        assert np.array_equal(el, kvbase + krow * kv_sr + 8 * (pc ^ sw(D, r)))
                        assert el.min() >= 0 and (el + 8).max() <= n_kv
                        assert krow.min() >= 0 and krow.max() < ln
            # compute tiles this wave keeps, and the mask decision
            kept_keys = set()
            rows = np.arange(qw0, qw0 + QW)
            valid = rows[rows < ln]
            for t in range(t_begin, t_end):
                for j in range(SUB):
                    k0 = t * KB + j * BN
                    if k0 >= kend:
                        break
                    if mode == "causal" and k0 > qw0 + QW - 1:
                        break
                    if mode == "window":
                        if k0 > qw0 + QW - 1 + wr:
                            break
                        if k0 + BN - 1 < qw0 - wl:
                            continue
                    need = k0 + BN > ln
                    if mode == "causal":
                        need |= k0 + BN - 1 > qw0
                    if mode == "window":
                        need |= (k0 < qw0 + QW - 1 - wl) or (k0 + BN - 1 > qw0 + wr)
                    keys = np.arange(k0, k0 + BN)
                    if not need and valid.size:
                        adm = (keys[None, :] < ln) & (keys[None, :] >= valid[:, None] - wl) & \
                              (keys[None, :] <= valid[:, None] + wr)
                        assert adm.all(), f"unmasked tile at key {k0} holds inadmissible keys"
                    kept_keys.update(keys.tolist())
            for i in valid.tolist():
                adm = range(max(0, i - wl), min(ln - 1, i + wr) + 1)
                missing = [k for k in adm if k not in kept_keys]
                assert not missing, f"row {i}: admissible keys {missing[:4]} never computed"
            # O and LSE stores
            for qb in range(QB):
                row = qw0 + 16 * qb + l16
                ok = row < ln
                if not ok.any():
                    continue
                for db in range(DB):
                    off = qbase + row * q_sr + 16 * db + 4 * g
                    assert off[ok].min() >= 0 and (off[ok] + 4).max() <= n_q
                lo = lbase + row
                assert lo[ok].min() >= 0 and lo[ok].max() < n_l


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
    # the kernel keeps one base per tensor and derives the k-step / column-block
    # offsets by XOR; that must equal the per-row formula
    rdK0, rdV0 = lds_read_bases(D, lane)
    for kk in range(DK):
        hoisted = 2 * (l16 * D + 8 * ((4 * kk + g) ^ swz_k(D, l16)))
        assert np.array_equal(rdK0 ^ (kk << 6), hoisted)
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
        assert np.array_equal(rdV0 ^ (db << 5), hoisted)
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


def _windows(S):
    out = []
    for wl, wr in ((0, 0), (1, 0), (3, 7), (64, 0), (100, 100), (255, 1), (0, 300), (S, 5), (7, S)):
        out.append((min(wl, S), min(wr, S)))
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", [1, 17, 64, 129, 300, 513, 1000])
def test_window_coverage_and_bounds(D, S):
    for window in _windows(S):
        emulate(1, 2, S, D, False, window=window)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 2), (8, 1), (6, 3)])
def test_gqa_bounds(D, H, H_kv):
    for S in (65, 300):
        for causal in (False, True):
            emulate(2, H, S, D, causal, H_kv=H_kv)
    emulate(1, H, 300, D, False, H_kv=H_kv, window=(20, 3))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [[5, 0, 17, 1, 9], [256, 255, 257], [1000], [0, 0, 3], [513, 64, 700, 1]])
def test_varlen_bounds(D, lens):
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    total = cu[-1]
    S = max(1, max(lens))
    for H, H_kv in ((2, 2), (4, 1)):
        for causal in (False, True):
            emulate(len(lens), H, S, D, causal, H_kv=H_kv, cu=cu, total=total)
        emulate(len(lens), H, S, D, False, H_kv=H_kv, cu=cu, total=total, window=(min(30, S), 0))


@pytest.mark.parametrize("D", [64, 128])
def test_malformed_sequence_tables_stay_in_bounds(D):
    """Entries outside [0, total], decreasing entries and lengths beyond the
    grid's longest sequence are clamped: no access leaves the tensors."""
    total = 300
    for cu, S in (([0, 500, 300], 300), ([-7, 100, 50, 300], 300), ([0, 300, 300], 64), ([10, 20, 400], 200),
                  ([0, 2**31 - 1, -2**31], 300)):
        emulate(len(cu) - 1, 2, S, D, False, cu=cu, total=total)
        emulate(len(cu) - 1, 2, S, D, True, cu=cu, total=total)


def _packed_keep_mask(word, thr):
    """The kernel's keep mask of one 32-bit word of two 16-bit draws, as its
    three packed 16-bit ops compute it: v_pk_sub_u16 with clamp (thr - draw,
    saturating at 0), v_pk_min_u16 with 1, v_pk_sub_u16 of 1 (wrapping)."""
    halves = np.stack([word & 0xFFFF, word >> 16]).astype(np.int64)
    over = np.maximum(thr - halves, 0)
    m = (np.minimum(over, 1) - 1) & 0xFFFF
    return (m[0] | (m[1] << 16)).astype(np.uint32)


@pytest.mark.parametrize("thr", [0, 1, 2, 6553, 32767, 32768, 65534, 65535])
def test_dropout_keep_mask_bit_trick(thr):
    """For every 16-bit draw in either half: 0xFFFF when draw >= thr (kept),
    0 otherwise, the other half independent."""
    d = np.arange(1 << 16, dtype=np.uint32)
    for other in (0, 1, thr, 0xFFFF):
        for word, shift in ((d | (np.uint32(other) << 16), 0), ((d << 16) | np.uint32(other), 16)):
            m = _packed_keep_mask(word, thr)
            assert np.array_equal((m >> shift) & 0xFFFF, np.where(d >= thr, 0xFFFF, 0).astype(np.uint32))
            assert np.all(((m >> (16 - shift)) & 0xFFFF) == (0xFFFF if other >= thr else 0))


def test_dropout_counter_names_the_register_key():
    """Element x of P^T register pb[qb][kc] of lane (l16, g) holds key
    j = k0 + 32kc + 16(x//4) + 4g + x%4 (the S^T accumulator order). The
    kernel computes one Philox group per lane, group(lane) = (k0 + 32kc)/8 +
    2(g&1) + (g>>1), and after swapping words 0<->2 and 1<->3 with the partner
    lane g^1 (v_permlane16_swap: rows 1 and 3 of the first operand trade with
    rows 0 and 2 of the second) reads element x from word (2(x//4) + (x%4)//2)
    of the swapped set, half x%2. That must be the definition's draw j%8 of
    group j//8."""
    lane = np.arange(64)
    g = lane >> 4
    partner = lane ^ 16
    for k0 in (0, 64, 4096 - 64, 123 * 64):
        for kc in range(2):
            group = (k0 + 32 * kc) // 8 + 2 * (g & 1) + (g >> 1)
            # symbolic words: (group, word index) held by each lane before the swaps
            own = [[(int(group[l]), w) for w in range(4)] for l in range(64)]
            odd_row = (g & 1) == 1
            s0 = [None] * 64
            s1 = [None] * 64
            t0 = [None] * 64
            t1 = [None] * 64
            for l in range(64):
                p = int(partner[l])
                # permlane16_swap(a=w0, b=w2): result[0] = a on even rows, partner's b on odd rows;
                # result[1] = partner's a on even rows, b on odd rows
                s0[l] = own[l][0] if not odd_row[l] else own[p][2]
                t0[l] = own[p][0] if not odd_row[l] else own[l][2]
                s1[l] = own[l][1] if not odd_row[l] else own[p][3]
                t1[l] = own[p][1] if not odd_row[l] else own[l][3]
            for l in range(64):
                w = [s0[l], s1[l], t0[l], t1[l]]
                for x in range(8):
                    key = k0 + 32 * kc + 16 * (x // 4) + 4 * int(g[l]) + x % 4
                    grp, word = w[2 * (x // 4) + (x % 4) // 2]
                    half = x % 2
                    t = key % 8
                    assert grp == key // 8, (k0, kc, l, x)
                    assert (word, half) == (t // 2, t % 2), (k0, kc, l, x)


@pytest.mark.parametrize("mode", ["none", "causal", "window"])
def test_mask_range_form_equals_the_per_key_rule(mode):
    """The kernel masks a tile's scores with one range test per element: per
    lane the admissible keys of row i are [lo, hi) (hi = min(len, i+1) causal,
    min(len, i+wr+1) windowed, len otherwise; lo = max(0, i-wl) windowed, else
    0), shifted by the lane's first key k0 + 4g; element offset o is kept when
    o < hi (unsigned o - lo < max(hi - lo, 0) windowed). That must equal the
    rule key < len and key <= i (causal) or i-wl <= key <= i+wr (window) for
    every key, including rows whose band misses the tile, ragged tails and the
    32x32x16 layout's offsets (32kb + 8t + e from k0 + 4h)."""
    g = np.random.Generator(np.random.PCG64(77 + len(mode)))
    offs16 = np.array([16 * kb + e for kb in range(4) for e in range(4)])
    offs32 = np.array([32 * kb + 8 * t + e for kb in range(2) for t in range(4) for e in range(4)])
    for _ in range(4000):
        ln = int(g.integers(1, 400))
        k0 = int(g.integers(0, (ln + 63) // 64)) * 64
        qrow = int(g.integers(0, ln + 40))
        wl, wr = int(g.integers(0, 300)), int(g.integers(0, 300))
        for lanebase, offs in ((4 * int(g.integers(0, 4)), offs16), (4 * int(g.integers(0, 2)), offs32)):
            base = k0 + lanebase
            hi = ln
            if mode == "causal":
                hi = min(hi, qrow + 1)
            if mode == "window":
                hi = min(hi, qrow + wr + 1)
            hi -= base
            lo = max(0, qrow - wl) - base if mode == "window" else 0
            width = max(hi - lo, 0)
            if mode == "window":
                keep = ((offs - lo) & 0xFFFFFFFF) < width
            else:
                keep = offs < hi
            key = base + offs
            rule = key < ln
            if mode == "causal":
                rule &= key <= qrow
            if mode == "window":
                rule &= (key >= qrow - wl) & (key <= qrow + wr)
            assert np.array_equal(keep, rule), (mode, ln, k0, qrow, wl, wr, lanebase)


# ---- the emulation against the kernel's own index code (fa2_index.h) ----

@pytest.fixture(scope="module")
def probe():
    """The host-only probe library over fa2_index.h, rebuilt when older than its sources."""
    from attention_forward_fa2_amd import build as b
    srcs = [b.INDEX_PROBE_SRC, os.path.join(b.CSRC, "fa2_index.h")]
    if not os.path.exists(b.INDEX_PROBE_LIB) or \
            os.path.getmtime(b.INDEX_PROBE_LIB) < max(os.path.getmtime(x) for x in srcs):
        b.build_index_probe()
    lib = ctypes.CDLL(b.INDEX_PROBE_LIB)
    i, ip, up = ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_uint32)
    lib.fa2_probe_swizzle.argtypes = [i, i, i]
    lib.fa2_probe_map_blocks.argtypes = [i] * 9 + [ip, i, i, i, i, ip, ip]
    lib.fa2_probe_map_blocks.restype = None
    lib.fa2_probe_lane_load_offsets.argtypes = [i] * 6 + [ip, up, up]
    lib.fa2_probe_lds_read_bases.argtypes = [i, i, up, up]
    return lib


def kernel_map(lib, mask, nqt, group, BH, serp=0, cu=None, lpt=0, S=0, total=0):
    """bh, qt per workgroup as the kernel's map_block computes them (-1: no work)."""
    BHkv = BH // group
    if cu is None:
        nb = BH * nqt
        cu_p, nseq = None, 0
    else:
        nb = -(-BHkv // 8) * 8 * nqt * group
        cu_arr = np.ascontiguousarray(cu, dtype=np.int32)
        cu_p, nseq = cu_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), len(cu_arr) - 1
    bh = np.empty(nb, dtype=np.int32)
    qt = np.empty(nb, dtype=np.int32)
    H = BH // nseq if cu is not None else BH       # query heads (read by the packed ranking only)
    lib.fa2_probe_map_blocks(mask, nqt, group, BH, BHkv, H, BH * nqt, serp, lpt, cu_p, nseq, total, S, nb,
                             bh.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
                             qt.ctypes.data_as(ctypes.POINTER(ctypes.c_int)))
    return bh, qt


def test_swizzles_equal_the_kernel(probe):
    for D in (64, 128):
        for r in range(512):
            assert probe.fa2_probe_swizzle(0, D, r) == swz_k(D, r)
            assert probe.fa2_probe_swizzle(1, D, r) == swz_v(D, r)


@pytest.mark.parametrize("BH", list(range(1, 41)) + [96, 192, 256])
@pytest.mark.parametrize("nqt", [1, 2, 3, 16, 33])
@pytest.mark.parametrize("mask", [0, 1, 2])
def test_dense_mapping_equals_the_kernel(probe, BH, nqt, mask):
    """The emulated mapping is the kernel's, for every workgroup; windows take
    the non-causal walk."""
    bh, qt = kernel_map(probe, mask, nqt, 1, BH)
    ebh, eqt = block_map(BH, nqt, mask == 1)
    assert np.array_equal(bh, ebh) and np.array_equal(qt, eqt)


@pytest.mark.parametrize("BHkv,group", [(8, 1), (16, 1), (8, 4), (24, 2), (12, 2), (1, 32), (32, 1), (4, 4)])
@pytest.mark.parametrize("nqt", [1, 5, 8, 16, 33, 64])
@pytest.mark.parametrize("serp", [0, 32])
def test_gqa_and_serpentine_mapping_equals_the_kernel(probe, BHkv, group, nqt, serp):
    BH = BHkv * group
    for mask in (0, 1):
        bh, qt = kernel_map(probe, mask, nqt, group, BH, serp=serp if mask == 1 else 0)
        ebh, eqt = block_map(BH, nqt, mask == 1, group, serp=serp if mask == 1 else 0)
        assert np.array_equal(bh, ebh) and np.array_equal(qt, eqt)


@pytest.mark.parametrize("nseq", [1, 2, 7, 24, 64, 70])
@pytest.mark.parametrize("H_kv,group", [(1, 1), (2, 4), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_mapping_equals_the_kernel(probe, nseq, H_kv, group, causal):
    """Packed launches, with the longest-first order (up to 64 sequences, lpt)
    and without it, on tables with ties, empty sequences and a malformed entry
    (the kernel clamps it)."""
    g = np.random.Generator(np.random.PCG64(nseq * 7 + H_kv + 100 * causal))
    lens = [int(x) if g.random() > 0.2 else int(g.choice([0, 5])) for x in g.integers(0, 3000, size=nseq)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total, S = int(cu[-1]), max(max(lens), 1)
    if nseq > 2:
        cu[2] = cu[1] - 3           # malformed: a start before the previous one
    BH, nqt = nseq * H_kv * group, 3
    lpt = int(nseq <= 64)
    bh, qt = kernel_map(probe, int(causal), nqt, group, BH, cu=cu, lpt=lpt, S=S, total=total)
    clamped = []
    for i in range(nseq):
        s0 = min(max(int(cu[i]), 0), total)
        clamped.append(min(min(max(int(cu[i + 1]), s0), total) - s0, S))
    ebh, eqt, ok = block_map_packed(BH, nqt, causal, group, clamped if lpt else None)
    assert np.array_equal(bh >= 0, ok)
    assert np.array_equal(bh[ok], ebh[ok]) and np.array_equal(qt[ok], eqt[ok])


@pytest.mark.parametrize("D,NW", [(64, 8), (64, 4), (128, 8), (128, 4)])
@pytest.mark.parametrize("kv_sr_heads", [1, 2, 8, 32])
def test_lane_load_offsets_equal_the_kernel(probe, D, NW, kv_sr_heads):
    """Dense (row stride D) and packed (row stride H_kv*D) K/V layouts."""
    kv_sr = kv_sr_heads * D
    row0 = ctypes.c_int()
    offK, offV = ctypes.c_uint32(), ctypes.c_uint32()
    for wave in range(NW):
        er, eK, eV = lane_load_offsets(D, NW, kv_sr, wave, np.arange(64))
        for lane in range(64):
            assert probe.fa2_probe_lane_load_offsets(D, NW, 0, kv_sr, wave, lane, ctypes.byref(row0),
                                                     ctypes.byref(offK), ctypes.byref(offV)) == 0
            assert (row0.value, offK.value, offV.value) == (er[lane], eK[lane], eV[lane])


@pytest.mark.parametrize("D", [64, 128])
def test_lds_read_bases_equal_the_kernel(probe, D):
    rk, rv = ctypes.c_uint32(), ctypes.c_uint32()
    eK, eV = lds_read_bases(D, np.arange(64))
    for lane in range(64):
        assert probe.fa2_probe_lds_read_bases(D, lane, ctypes.byref(rk), ctypes.byref(rv)) == 0
        assert (rk.value, rv.value) == (eK[lane], eV[lane])
