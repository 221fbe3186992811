"""LDS layout of the 16-bit forward kernel's K/V stages, checked on the host.

At d <= 128 a tile of 64 key rows of 2d bytes sits in LDS unpadded, and
16-byte chunk c of row r is stored at chunk c ^ swz(r). At d = 256 rows are
padded instead (K rows 2d + 16 bytes apart, V rows 2d + 64). These tests
restate, in Python, the kernel's address formulas (the copy map of tile_src,
the per-lane offsets of the K reads and of the transposed V reads in
fwd16_tile) and check that

- the copies of the 4 waves write every data chunk of a tile exactly once,
  each from its own (row, chunk) of the source (at d = 256 the remaining
  slots are padding or filler, which fetch nothing);
- every K read (16 bytes) and V read (8 bytes) finds the logical row and
  columns the MFMA operand needs;
- no 16-lane ds_read_b128 phase and no 32-lane ds_read_b64_tr_b16 phase
  touches a bank twice (64 banks of 4 bytes).
"""

import pytest

KBC = 64  # keys per tile
WAVES = 4


def swizzled(d):
    return d <= 128


def strides(d):
    """LDS row strides of K and V."""
    if swizzled(d):
        return 2 * d, 2 * d
    return 2 * d + 16, 2 * d + 64


def tile_bytes(stride):
    return (KBC * stride + 4095) // 4096 * 4096


def swz(d, r):
    if d == 64:
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
    return ((r & 3) << 2) | ((r >> 2) & 3)


def sigma(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def slot_to_logical(d, stride, t):
    """LDS slot t (16 bytes) -> (row, logical chunk) it holds, or None for a
    pad or filler slot."""
    nch = stride // 16
    r, p = divmod(t, nch)
    if swizzled(d):
        return r, p ^ swz(d, r)
    if p >= d // 8 or r >= KBC:
        return None
    return r, p


def addr_to_logical(d, stride, a):
    """LDS byte address inside a tile -> (row, logical byte column)."""
    rc = slot_to_logical(d, stride, a // 16)
    assert rc is not None, "read of a pad slot"
    return rc[0], 16 * rc[1] + a % 16


def k_offsets(d, lane):
    """Per-lane K read offsets of k-steps s = 0 .. d/16 - 1 (keys 0..31)."""
    n, hh = lane & 31, lane >> 5
    sk, _ = strides(d)
    if swizzled(d):
        ksw = swz(d, sigma(n))
        return [sigma(n) * sk + 16 * ((2 * s + hh) ^ ksw) for s in range(d // 16)]
    return [sigma(n) * sk + 16 * hh + 32 * s for s in range(d // 16)]


def v_offset(d, lane, cc, t, h):
    vb, vj = lane >> 4, lane & 15
    vr = 8 * (vb >> 1) + (vj >> 2)
    _, sv = strides(d)
    if swizzled(d):
        vx = 2 * (vb & 1) + ((vj & 3) >> 1)
        return 16 * cc * sv + (vr + 4 * h) * sv + 16 * ((4 * t + vx) ^ swz(d, vr + 4 * h)) + 8 * (vj & 1)
    return vr * sv + 32 * (vb & 1) + 8 * (vj & 3) + 4 * h * sv + 16 * cc * sv + 64 * t


def banks(addr, nbytes):
    return {((addr + b) // 4) % 64 for b in range(0, nbytes, 4)}


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("which", [0, 1])  # K, V
def test_copies_cover_every_chunk_once(d, which):
    stride = strides(d)[which]
    tile = tile_bytes(stride)
    if swizzled(d):
        assert tile == KBC * 2 * d  # no padding, no filler
    per_wave = tile // 4096
    seen = {}
    for w in range(WAVES):
        for i in range(per_wave):
            for lane in range(64):
                t = 64 * (w + 4 * i) + lane  # LDS slot this lane writes
                assert t not in seen
                seen[t] = slot_to_logical(d, stride, t)
    assert sorted(seen) == list(range(tile // 16))
    data = sorted(v for v in seen.values() if v is not None)
    assert data == [(r, c) for r in range(KBC) for c in range(d // 8)]


@pytest.mark.parametrize("d", [64, 128, 256])
def test_k_reads_find_their_operand(d):
    sk, _ = strides(d)
    for lane in range(64):
        n, hh = lane & 31, lane >> 5
        for s, off in enumerate(k_offsets(d, lane)):
            for half in range(2):
                a = off + 32 * sk * half
                # MFMA row n holds key sigma(n) (+32), 8 values from column 16s + 8hh
                assert addr_to_logical(d, sk, a) == (sigma(n) + 32 * half, 2 * (16 * s + 8 * hh))
                assert addr_to_logical(d, sk, a + 15)[1] == 2 * (16 * s + 8 * hh) + 15


@pytest.mark.parametrize("d", [64, 128, 256])
def test_v_reads_find_their_operand(d):
    _, sv = strides(d)
    for lane in range(64):
        vb, vj = lane >> 4, lane & 15
        for cc in range(4):
            for t in range(d // 32):
                for h in range(2):
                    r, col = addr_to_logical(d, sv, v_offset(d, lane, cc, t, h))
                    want_r = 16 * cc + 8 * (vb >> 1) + (vj >> 2) + 4 * h
                    want_col = 2 * (32 * t + 16 * (vb & 1) + 4 * (vj & 3))
                    assert (r, col) == (want_r, want_col)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_reads_are_bank_conflict_free(d):
    sk, _ = strides(d)
    for s in range(d // 16):
        for half in range(2):
            for ph in range(4):  # ds_read_b128: 16-lane phases
                used = []
                for lane in range(16 * ph, 16 * ph + 16):
                    used += list(banks(k_offsets(d, lane)[s] + 32 * sk * half, 16))
                assert len(set(used)) == 64, (d, s, half, ph)
    for cc in range(4):
        for t in range(d // 32):
            for h in range(2):
                for ph in range(2):  # ds_read_b64_tr_b16: 32-lane phases
                    used = []
                    for lane in range(32 * ph, 32 * ph + 32):
                        used += list(banks(v_offset(d, lane, cc, t, h), 8))
                    assert len(set(used)) == 64, (d, cc, t, h, ph)


def test_a_padding_free_layout_needs_the_swizzle():
    """Negative control: without the swizzle the K phases conflict."""
    d = 128
    used = []
    for lane in range(16):
        n = lane & 31
        used += list(banks(sigma(n) * 2 * d, 16))
    assert len(set(used)) < 64
