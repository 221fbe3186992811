"""CPU checks of the strided entry points' host-side validation
(fa_fwd_strided_check / fa_bwd_strided_check make no HIP call).

The overlap rules are pinned against brute force: for random layouts built
from slices of shared buffers, every byte each view touches is marked in an
array, and whenever the library accepts a layout the outputs must share no
byte with any other operand (soundness). The layouts the user calls produce
(packed [B, N, 3, H, d], [B, N, H, d], contiguous [B, H, N, d]) must be
accepted (no false alarm on them)."""

import itertools

import numpy as np
import pytest

import transformer_exact_attention_flashattention_amd as fa
from transformer_exact_attention_flashattention_amd import build as fabuild

OK, SHAPE, ALIGN, ARG = 0, -2, -5, -6


@pytest.fixture(scope="module", autouse=True)
def built():
    if not fabuild.is_built():
        fabuild.build()
    return fa.lib()


def fwd_check(ptrs, strides, B, H, N, d=64, dtype=fa.FA_BF16, lse=0x7000_0000):
    q, k, v, o = ptrs
    return fa.fa_fwd_strided_check(q, k, v, o, lse, strides, B, H, N, d, 0.125, 0, -1, -1, dtype)


def bwd_check(ptrs, strides, B, H, N, d=64, lse=0x7000_0000, delta=0x7800_0000):
    q, k, v, o, do, dq, dk, dv = ptrs
    return fa.fa_bwd_strided_check(q, k, v, o, lse, do, dq, dk, dv, delta, strides, B, H, N, d, 0.125, 0,
                                   -1, -1, fa.FA_BF16)


def packed(base, B, N, H, d, slot, nslots=3, esz=2):
    """(pointer, strides) of slot `slot` of a [B, N, nslots, H, d] tensor."""
    return base + slot * H * d * esz, [N * nslots * H * d, d, nslots * H * d]


def bnhd(base, B, N, H, d):
    return base, [N * H * d, d, H * d]


def bhnd(base, B, N, H, d):
    return base, [H * N * d, N * d, d]


# ------------------------------------------------- layouts that must pass --

@pytest.mark.parametrize("B,H,N,d", [(2, 12, 256, 64), (1, 3, 5, 128), (3, 1, 7, 256), (2, 2, 1, 64)])
def test_packed_qkv_with_separate_output_accepted(B, H, N, d):
    base = 0x100_0000
    ps, ss = zip(*(packed(base, B, N, H, d, i) for i in range(3)))
    o, so = bnhd(0x4000_0000, B, N, H, d)
    assert fwd_check(list(ps) + [o], sum(ss, []) + so, B, H, N, d) == OK


@pytest.mark.parametrize("B,H,N,d", [(2, 12, 256, 64), (1, 3, 5, 128), (4, 2, 9, 64)])
def test_packed_gradient_accepted(B, H, N, d):
    q = [packed(0x100_0000, B, N, H, d, i) for i in range(3)]
    g = [packed(0x2000_0000, B, N, H, d, i) for i in range(3)]
    o = bnhd(0x4000_0000, B, N, H, d)
    do = bnhd(0x5000_0000, B, N, H, d)
    items = q + [o, do] + g
    ptrs = [p for p, _ in items]
    strides = sum((s for _, s in items), [])
    assert bwd_check(ptrs, strides, B, H, N, d) == OK


def test_output_slot_inside_a_packed_buffer_accepted():
    # o written into slot 3 of a [B, N, 4, H, d] buffer whose slots 0..2 are q, k, v
    B, H, N, d = 2, 4, 33, 64
    items = [packed(0x100_0000, B, N, H, d, i, nslots=4) for i in range(4)]
    assert fwd_check([p for p, _ in items], sum((s for _, s in items), []), B, H, N, d) == OK


def test_contiguous_and_null_strides_agree():
    B, H, N, d = 2, 3, 50, 128
    ptrs = [0x100_0000 + i * 0x100_0000 for i in range(4)]
    strides = sum((bhnd(0, B, N, H, d)[1] for _ in range(4)), [])
    assert fwd_check(ptrs, strides, B, H, N, d) == OK
    assert fwd_check(ptrs, None, B, H, N, d) == OK


def test_inputs_may_alias_and_broadcast():
    B, H, N, d = 1, 4, 20, 64
    q, sq = bhnd(0x100_0000, B, N, H, d)
    kv = [0x200_0000, [0, 0, d]]  # one K = V shared by all heads (head stride 0)
    o, so = bhnd(0x300_0000, B, N, H, d)
    assert fwd_check([q, kv[0], kv[0], o], sq + kv[1] + kv[1] + so, B, H, N, d) == OK
    # q, k, v all the same tensor
    assert fwd_check([q, q, q, o], sq * 3 + so, B, H, N, d) == OK


def test_unused_strides_of_extent_one_ignored():
    # B = 1, N = 1: batch and row strides are never used (any value passes)
    d = 64
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    strides = [-5, d, 3] * 4
    assert fwd_check(ptrs, strides, 1, 2, 1, d) == OK


# ----------------------------------------------- layouts that must fail --

def four(strides_q, **kw):
    B, H, N, d = kw.get("B", 1), kw.get("H", 2), kw.get("N", 10), 64
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    rest = [H * N * d, N * d, d]
    return fwd_check(ptrs, list(strides_q) + rest * 3, B, H, N, d)


@pytest.mark.parametrize("sq,code", [
    ((-640 * 2, 640, 64), SHAPE),    # negative batch stride
    ((1280, -640, 64), SHAPE),       # negative head stride
    ((1280, 640, 32), SHAPE),        # rows overlap (row stride < d)
    ((1280, 640, 0), SHAPE),
    ((1280, 640, (1 << 24) + 8), SHAPE),  # row stride above 32 MiB in bytes
    ((1280, 640, 68), ALIGN),        # 136-byte rows: not 16-byte aligned
    ((1280, 644, 64), ALIGN),
    ((1284, 640, 64), ALIGN),
])
def test_bad_strides(sq, code):
    assert four(sq, B=2) == code


def test_output_overlapping_an_input_rejected():
    B, H, N, d = 2, 4, 16, 64
    items = [packed(0x100_0000, B, N, H, d, i) for i in range(3)]
    ptrs = [p for p, _ in items]
    strides = sum((s for _, s in items), [])
    for slot in range(3):  # o in the slot of q, k or v
        assert fwd_check(ptrs + [ptrs[slot]], strides + items[slot][1], B, H, N, d) == ARG
    # o shifted by 16 bytes into q's slot: partial overlap
    assert fwd_check(ptrs + [ptrs[0] + 16], strides + items[0][1], B, H, N, d) == ARG


def test_self_overlapping_output_rejected():
    B, H, N, d = 1, 2, 10, 64
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    good = [H * N * d, N * d, d]
    for so in ([0, 0, d], [0, d, d], [0, 2 * d, d]):  # heads on the same rows / interleaved
        assert fwd_check(ptrs, good * 3 + so, B, H, N, d) == ARG


def test_lse_overlap_rejected():
    B, H, N, d = 1, 2, 10, 64
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    assert fwd_check(ptrs, None, B, H, N, d, lse=0x300_0000 + 64) == ARG
    assert fwd_check(ptrs, None, B, H, N, d, lse=0x400_0000) == ARG


def test_gradients_overlapping_rejected():
    B, H, N, d = 2, 3, 40, 64
    q = [packed(0x100_0000, B, N, H, d, i) for i in range(3)]
    o = bnhd(0x4000_0000, B, N, H, d)
    do = bnhd(0x5000_0000, B, N, H, d)
    g = [packed(0x2000_0000, B, N, H, d, i) for i in range(3)]
    def run(items, **kw):
        return bwd_check([p for p, _ in items], sum((s for _, s in items), []), B, H, N, d, **kw)
    assert run(q + [o, do] + g) == OK
    assert run(q + [o, do] + [g[0], g[0], g[2]]) == ARG   # dq and dk in one slot
    assert run(q + [o, do] + [q[0], g[1], g[2]]) == ARG   # dq over q
    assert run(q + [o, do] + [g[0], g[1], o]) == ARG      # dv over o
    assert run(q + [o, do] + g, delta=0x2000_0000) == ARG  # delta inside the gradient
    assert run(q + [o, do] + g, delta=0x7000_0000) == ARG  # delta on lse
    assert run(q + [o, o] + g) == OK                       # inputs may alias (do = o)


def test_strides_array_length_checked():
    with pytest.raises(ValueError):
        fa.fa_fwd_strided_check(1, 2, 3, 4, 5, [1, 2, 3], 1, 1, 1, 64, 1.0, 0, -1, -1, 1)


def test_strided_entry_shares_the_checks():
    # failing checks return before any HIP call
    B, H, N, d = 2, 4, 16, 64
    items = [packed(0x100_0000, B, N, H, d, i) for i in range(3)]
    ptrs = [p for p, _ in items]
    strides = sum((s for _, s in items), [])
    assert fa.fa_fwd_strided(*ptrs, ptrs[1], 0x7000_0000, strides + items[1][1], B, H, N, d, 0.125, 0, -1, -1,
                             fa.FA_BF16) == ARG


# ------------------------------------------------ brute-force soundness --

def touched(ptr, strides, B, H, N, d, esz, lo, size):
    """Boolean map of the bytes [lo, lo + size) a view touches."""
    m = np.zeros(size, dtype=bool)
    for b, h, n in itertools.product(range(B), range(H), range(N)):
        s = ptr + esz * (b * strides[0] + h * strides[1] + n * strides[2]) - lo
        m[s:s + d * esz] = True
    return m


def self_overlaps(ptr, strides, B, H, N, d, esz):
    starts = sorted(ptr + esz * (b * strides[0] + h * strides[1] + n * strides[2])
                    for b, h, n in itertools.product(range(B), range(H), range(N)))
    return any(b - a < d * esz for a, b in zip(starts, starts[1:]))


def random_layout(rng, B, H, N, d):
    """q, k, v, o as slots (or byte-shifted slots) of one or two packed
    buffers with a random dimension order, or head-broadcast inputs."""
    esz = 2
    nslots = int(rng.integers(1, 5))
    order = list(rng.permutation(4))  # memory order of (B, N, slot, H), slowest first
    ext = {0: B, 1: N, 2: nslots, 3: H}
    stride = {}
    acc = d
    for dim in reversed(order):
        stride[dim] = acc
        acc *= ext[dim]
    bases = [0x10_0000, 0x10_0000 + int(rng.integers(0, 3)) * acc * esz // 2 // 16 * 16]
    ptrs, strides = [], []
    for _ in range(4):
        base = bases[int(rng.integers(0, 2))]
        slot = int(rng.integers(0, nslots))
        shift = 16 * int(rng.integers(0, 3)) if rng.random() < 0.3 else 0
        ptrs.append(base + esz * slot * stride[2] + shift)
        sh = 0 if rng.random() < 0.1 else stride[3]
        strides += [stride[0], sh, stride[1]]
    return ptrs, strides


def test_bruteforce_soundness_of_overlap_rules():
    rng = np.random.default_rng(2024)
    accepted = rejected = 0
    for trial in range(400):
        B, H, N = (int(x) for x in rng.integers(1, 4, size=3))
        d, esz = 64, 2
        ptrs, strides = random_layout(rng, B, H, N, d)
        st = fwd_check(ptrs, strides, B, H, N, d)
        assert st in (OK, ARG, ALIGN, SHAPE), st
        if st != OK:
            rejected += 1
            continue
        accepted += 1
        lo = min(ptrs)
        size = max(p + esz * (B * s[0] + H * s[1] + N * s[2] + d) for p, s in
                   zip(ptrs, (strides[i:i + 3] for i in range(0, 12, 3)))) - lo
        maps = [touched(p, strides[3 * i:3 * i + 3], B, H, N, d, esz, lo, size) for i, p in enumerate(ptrs)]
        for i in range(3):
            assert not (maps[3] & maps[i]).any(), f"trial {trial}: o overlaps input {i} but was accepted"
        assert not self_overlaps(ptrs[3], strides[9:12], B, H, N, d, esz), f"trial {trial}: o overlaps itself"
    # the generator produces both outcomes in quantity
    assert accepted > 50 and rejected > 50, (accepted, rejected)


# ------------------------------------------------------------- split-KV --

def splitkv(ws, ws_bytes, splits, B=1, H=2, N=300, d=64):
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    return fa.fa_fwd_splitkv(*ptrs, 0x7000_0000, None, ws, ws_bytes, splits, B, H, N, d, 0.125, 0, -1, -1,
                             fa.FA_BF16)


def test_splitkv_workspace_size():
    assert fa.splitkv_workspace_bytes(2, 3, 100, 128, 4) == 4 * 4 * 2 * 3 * 100 * 129
    assert fa.splitkv_workspace_bytes(2, 3, 100, 128, 1) == 0
    for bad in (0, 65, -1):
        with pytest.raises(fa.FaError):
            fa.splitkv_workspace_bytes(1, 1, 10, 64, bad)


def test_splitkv_heuristic():
    # large grids are not split
    assert fa.splitkv_num_splits(1, 16, 16384, 256, True) == 1
    assert fa.splitkv_num_splits(1, 128, 2048, 128, True) == 1
    # one long head: split, at most 16 parts
    s = fa.splitkv_num_splits(1, 1, 16384, 128, True)
    assert 2 <= s <= 16
    # every answer is within 1 .. 16 and 0 sizes give 1
    assert fa.splitkv_num_splits(0, 4, 100, 64) == 1
    for B, H, N, d in itertools.product((1, 2), (1, 3), (1, 65, 1000, 9000), (64, 128, 256)):
        assert 1 <= fa.splitkv_num_splits(B, H, N, d, False) <= 16


@pytest.mark.parametrize("ws,ws_bytes,splits,code", [
    (0x5000_0000, 1 << 30, -1, ARG), (0x5000_0000, 1 << 30, 65, ARG),
    (0, 1 << 30, 2, -1),                # no workspace
    (0x5000_0008, 1 << 30, 2, ALIGN),   # misaligned workspace
    (0x5000_0000, 1000, 2, ARG),        # too small
    (0x200_0000 - 64, 1 << 30, 2, ARG),  # overlaps k
    (0x7000_0000 - 256, 1 << 30, 3, ARG),  # overlaps lse
])
def test_splitkv_errors(ws, ws_bytes, splits, code):
    assert splitkv(ws, ws_bytes, splits) == code


# ----------------------------------------------- queries against a cache --

def fwd_kv(N, Nk, causal=0, left=-1, right=-1, B=1, H=2, d=64):
    ptrs = [0x100_0000, 0x200_0000, 0x300_0000, 0x400_0000]
    return fa.fa_fwd_kv(*ptrs, 0x7000_0000, None, None, 0, 1, B, H, N, Nk, d, 0.125, causal, left, right,
                        fa.FA_BF16)


@pytest.mark.parametrize("N,Nk,causal,left,right,code", [
    (5, -1, 0, -1, -1, SHAPE),
    (5, 1 << 30, 0, -1, -1, SHAPE),
    (5, 0, 0, -1, -1, ARG),       # no key at all
    (8, 4, 1, -1, -1, ARG),       # causal: rows 0..3 sit before the first key
    (8, 4, 0, 2, -1, ARG),        # window: the same
    (8, 4, 0, -1, 0, ARG),
    (0, 0, 1, -1, -1, OK),        # nothing to do
])
def test_fwd_kv_checks(N, Nk, causal, left, right, code):
    assert fwd_kv(N, Nk, causal, left, right) == code


def test_fwd_kv_num_splits_for_decode():
    # one query per head against a long cache: about one workgroup per
    # compute unit (256), at most 64 parts, at least 16 key tiles per part
    assert fa.splitkv_num_splits(1, 32, 1, 128, True, Nk=32768) == 8
    assert fa.splitkv_num_splits(1, 4, 1, 128, True, Nk=262144) == 64
    assert fa.splitkv_num_splits(8, 32, 1, 128, True, Nk=4096) == 1
    assert fa.splitkv_num_splits(1, 32, 1, 128, True, Nk=256) == 1
    assert fa.splitkv_num_splits(4, 64, 2048, 128, True, Nk=4096) == 1
    # matrix-core bound shapes keep filling the resident slots (at most 16)
    assert fa.splitkv_num_splits(1, 1, 16384, 128, True) == 4


# ------------------------------------------- the allocation-free forward --

def fwd_noalloc(N, Nk, splits, causal=0, B=1, H=2, d=64, step=0x100_0000):
    ptrs = [step, 2 * step, 3 * step, 4 * step, 5 * step]
    return fa.fa_fwd_kv_noalloc(*ptrs, None, splits, B, H, N, Nk, d, 0.125, causal, -1, -1, fa.FA_BF16)


def test_noalloc_rejects_partials_beyond_its_scratch_before_any_hip_call():
    # 16 parts of 64 heads x 4096 rows x (256 + 1) floats: 4.3 GB > 64 MiB
    assert fwd_noalloc(4096, 4096, 16, B=1, H=64, d=256, step=0x1000_0000) == -8
    # one byte-count past the limit is refused, the largest that fits is not checked here (it would launch)
    need = 4 * 2 * 1 * 64 * 1024 * (256 + 1)  # 2 parts, 64 heads, 1024 rows, d = 256
    assert need > fa.NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(1024, 1024, 2, H=64, d=256, step=0x1000_0000) == -8
    assert "scratch" in fa.strerror(-8)


@pytest.mark.parametrize("N,Nk,splits,causal,code", [
    (5, 100, -1, 0, ARG), (5, 100, 65, 0, ARG),
    (5, 0, 2, 0, ARG),            # no key at all
    (8, 4, 2, 1, ARG),            # causal: rows before the first key
    (5, -1, 2, 0, SHAPE),
    (0, 0, 2, 1, OK),             # nothing to do
])
def test_noalloc_shares_the_checks(N, Nk, splits, causal, code):
    assert fwd_noalloc(N, Nk, splits, causal) == code
