"""LDS bank model of the bf16 kernels' K/V tile reads (host logic, no GPU).

The model, fitted to conflict counts measured on gfx950 (SQ_LDS_BANK_CONFLICT of probe kernels
that repeat one read kind at the attention kernel's address pattern):
- LDS has 64 banks of 4 bytes; a wave-wide read is served in passes of 32 lanes, and a pass
  costs as many cycles as the largest number of dwords that its lanes ask of one bank;
- a 16-byte read (ds_read_b128) also pays when a row's run of 16-byte pieces (the lanes that
  read one row, 4 consecutive chunks here) starts 16 but not 32 bytes aligned.

It reproduces the measured cycles per instruction for row strides of 10 to 17 chunks of 16 bytes
(K operand reads: 0 at even strides not divisible by 4, about 4 at odd strides and at 12, about
28 at 16; 8-byte tail reads: 0 at odd strides, 2 at 10 and 14, 6 at 12, 30 at 16), and the test
checks that the layout the kernel uses -- K rows of KCH chunks with KCH the smallest count
>= DK/8 with KCH % 4 == 2, the two tail chunks swapped in rows with bit 3 set, V rows of 10
(18 for head_dim 128) chunks -- has no conflict in any of the three read kinds.  The layout
constants are restated here from the kernel's configuration (Bf16Cfg, load_k, load_v,
Dma::lane_offset).
"""
from __future__ import annotations

import pytest

BANKS, PASS = 64, 32


def pass_cycles(dword_addrs_per_lane):
    """Cycles of one wave-wide read: per pass of 32 lanes, the largest dword count on one bank."""
    total = 0
    for p0 in range(0, 64, PASS):
        per_bank = {}
        for lane in range(p0, p0 + PASS):
            for a in dword_addrs_per_lane[lane]:
                per_bank[a % BANKS] = per_bank.get(a % BANKS, 0) + 1
        total += max(per_bank.values())
    return total


def misaligned_16(byte_addrs):
    """Some row's run of 16-byte reads (lanes g = 0..3 of row c read 4 consecutive chunks)
    starts 16 but not 32 bytes aligned: its first lane is g = 0."""
    return any(byte_addrs[lane] % 32 == 16 for lane in range(16))


def kch_of(head_dim):
    nk32, tail = head_dim // 32, 1 if head_dim % 32 else 0
    dk = nk32 * 32 + 16 * tail
    return (dk // 8 + 1) // 4 * 4 + 2


def vch_of(head_dim):
    return 10 if head_dim <= 80 else 18


def k_operand_read(stride_chunks, kb, ks):
    """ds_read_b128 of the K operand: lane (c, g) reads row kb*16 + c, elements ks*32 + 8g .. +8."""
    addrs, byte_addrs = [], []
    for lane in range(64):
        g, c = lane >> 4, lane & 15
        b = (kb * 16 + c) * stride_chunks * 16 + (ks * 32 + 8 * g) * 2
        byte_addrs.append(b)
        addrs.append([b // 4 + i for i in range(4)])
    return addrs, byte_addrs


def k_tail_read(stride_chunks, kb, nk32, swizzle):
    """ds_read_b64 of the 16-deep tail: lane (c, g) reads elements nk32*32 + 4g .. +4 of row
    kb*16 + c, at the swapped chunk in rows with bit 3 set when `swizzle`."""
    addrs = []
    for lane in range(64):
        g, c = lane >> 4, lane & 15
        col = (4 * g) ^ (c & 8) if swizzle else 4 * g
        b = (kb * 16 + c) * stride_chunks * 16 + (nk32 * 32 + col) * 2
        addrs.append([b // 4, b // 4 + 1])
    return addrs


def v_transposed_read(stride_chunks, db, half):
    """ds_read_b64_tr_b16 of V^T: lane (g, i) reads 8 bytes of row half*16 + 4g + i//4 at
    element db*16 + 4*(i % 4)."""
    addrs = []
    for lane in range(64):
        g, i = lane >> 4, lane & 15
        b = (half * 16 + 4 * g + (i >> 2)) * stride_chunks * 16 + (db * 16 + 4 * (i & 3)) * 2
        addrs.append([b // 4, b // 4 + 1])
    return addrs


def k_operand_conflicts(stride):
    base = min(pass_cycles(k_operand_read(s, 0, 0)[0]) for s in (10, 14, 18))  # the conflict-free cost
    addrs, byte_addrs = k_operand_read(stride, 0, 0)
    return pass_cycles(addrs) - base + (4 if misaligned_16(byte_addrs) else 0)


def k_tail_conflicts(stride, swizzle=False):
    base = pass_cycles(k_tail_read(11, 0, 2, False))  # odd strides: measured conflict-free
    return pass_cycles(k_tail_read(stride, 0, 2, swizzle)) - base


# measured conflict cycles per instruction (probe kernels, head_dim 80 address pattern)
MEASURED = {10: (0.0, 1.97), 11: (3.94, 0.0), 12: (3.94, 5.91), 13: (3.94, 0.0), 14: (0.0, 1.97),
            15: (3.94, 0.0), 16: (27.6, 29.5), 17: (3.94, 0.0)}


@pytest.mark.parametrize("stride", sorted(MEASURED))
def test_model_reproduces_the_measured_conflicts(stride):
    m128, m64 = MEASURED[stride]
    assert abs(k_operand_conflicts(stride) - m128) <= 0.5
    assert abs(k_tail_conflicts(stride) - m64) <= 0.5


@pytest.mark.parametrize("head_dim", [64, 72, 80, 128])
def test_kernel_layout_is_conflict_free(head_dim):
    kch, vch = kch_of(head_dim), vch_of(head_dim)
    assert kch % 4 == 2 and kch * 8 >= head_dim
    nk32, tail = head_dim // 32, head_dim % 32 != 0
    for kb in range(2):
        for ks in range(nk32):
            addrs, byte_addrs = k_operand_read(kch, kb, ks)
            assert not misaligned_16(byte_addrs)
            assert pass_cycles(addrs) == pass_cycles(k_operand_read(10, 0, 0)[0])
        if tail:
            assert kch == nk32 * 4 + 2  # the swizzle swaps the last two chunks of a row
            assert pass_cycles(k_tail_read(kch, kb, nk32, True)) == pass_cycles(k_tail_read(11, 0, 2, False))
    dv = (head_dim + 15) // 16 * 16
    assert vch * 8 >= dv
    ideal = pass_cycles(v_transposed_read(10, 0, 0))
    for db in range(dv // 16):
        for half in range(2):
            assert pass_cycles(v_transposed_read(vch, db, half)) == ideal


def test_the_tail_swizzle_is_what_removes_the_tail_conflict():
    assert k_tail_conflicts(10, swizzle=False) == 2
    assert k_tail_conflicts(10, swizzle=True) == 0


def test_swizzled_tail_reads_the_right_elements():
    # rows with bit 3 set hold chunk 9 at position 8 and chunk 8 at position 9 (head_dim 80):
    # the element a lane reads must be the one it wants, for every lane and row
    kch, nk32 = kch_of(80), 2
    for c in range(16):
        stored = {}  # position (element offset in the row) -> global element
        for pos_chunk in range(kch):
            src_chunk = pos_chunk ^ 1 if (pos_chunk >= nk32 * 4 and c & 8) else pos_chunk
            for e in range(8):
                stored[pos_chunk * 8 + e] = src_chunk * 8 + e
        for g in range(4):
            col = nk32 * 32 + ((4 * g) ^ (c & 8))
            assert [stored[col + e] for e in range(4)] == [nk32 * 32 + 4 * g + e for e in range(4)]
