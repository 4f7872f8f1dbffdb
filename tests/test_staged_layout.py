"""CPU model of the staged activation layout's index arithmetic.

The staging helper stores float4 number i of a k-vector as one 32-bit word
per byte plane, at word i + 4*(i // 32) of a plane of n4 + n4/8 words
(n4 = k/4; 16 bytes of padding after every 128 inputs), and the group's
scale and sum at index i // (GROUP/4) of two f32 tables after the planes.
This model checks that every in-range float4 lands in its own plane at a
distinct word, and shows what an out-of-range float4 (i >= n4) would hit if
it were stored: the next plane, or for the last plane the scale and sum
tables.  That is why the helper stores nothing for i >= n4.

It is also the cause of a wrong-result variant tried in the fused tail +
gate/up kernel: encoding all four register slots of each tail thread and
storing them, slots past the row included.  At k = 768 the tail runs one
wave (64 threads x 4 slots = 256 float4 for n4 = 192), so slots 192..255
were stored: into planes 1 and 2 and, from the last plane, over
scale[24..31] -- which is sum[0..7], the Q4_K group sums of the min term --
and the sums that follow.  x itself (written from registers) stayed
identical while mid changed, as was observed.
"""
import numpy as np

LIMBS = 3


def layout(k, group):
    n4 = k // 4
    pw = n4 + n4 // 8                      # words per plane
    planes = LIMBS * pw                    # words of all planes
    scale0, sum0 = planes, planes + k // group
    end = sum0 + k // group
    return n4, pw, scale0, sum0, end


def stores(i, k, group):
    """Word addresses (in 4-byte words from the staged form's start) an
    unguarded store of float4 i would write: one per plane, plus the scale
    and sum of its group when i leads the group."""
    n4, pw, scale0, sum0, _ = layout(k, group)
    wi = i + ((i >> 5) << 2)
    out = [("plane", l, l * pw + wi) for l in range(LIMBS)]
    tpg = group // 4
    if i % tpg == 0:
        g = i // tpg
        out += [("scale", g, scale0 + g), ("sum", g, sum0 + g)]
    return out


def region(addr, k, group):
    n4, pw, scale0, sum0, end = layout(k, group)
    if addr < scale0:
        return ("plane", addr // pw)
    if addr < sum0:
        return ("scale", addr - scale0)
    if addr < end:
        return ("sum", addr - sum0)
    return ("past", addr - end)


def test_in_range_float4_land_in_their_own_plane_and_tables():
    for group in (16, 32):
        for k in (256, 768, 6656, 19968):
            n4 = k // 4
            seen = set()
            for i in range(n4):
                for kind, idx, addr in stores(i, k, group):
                    assert addr not in seen, (k, group, i)
                    seen.add(addr)
                    got = region(addr, k, group)
                    if kind == "plane":
                        assert got == ("plane", idx), (k, group, i, got)
                    else:
                        assert got == (kind, idx), (k, group, i, got)
            # the padding words (4 per 32 float4) are the only words not written
            _, pw, scale0, _, end = layout(k, group)
            assert len(seen) == end - LIMBS * (pw - n4)


def test_out_of_range_float4_would_overwrite_next_plane_and_group_sums():
    k, group = 768, 32                      # one 64-thread tail wave, 4 slots each
    n4 = k // 4
    hit = set()
    for i in range(n4, 256):
        for kind, idx, addr in stores(i, k, group):
            hit.add(region(addr, k, group))
    assert ("plane", 1) in hit and ("plane", 2) in hit
    sums = sorted(j for r, j in hit if r == "sum")
    assert sums[:8] == list(range(8)), sums      # group sums 0..7 of the min term
    assert any(r == "scale" for r, _ in hit)
