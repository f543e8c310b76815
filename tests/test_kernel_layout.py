"""Host-side checks of address identities the prefill kernel relies on.

Where one wave covers all of D, the kernel keeps only the first copy op's
per-lane offset and derives op i's as (off0 ^ dx_i) + drow_i with dx_i and
drow_i the same for every lane of the wave.  That needs the swizzle of op i's
rows to differ from op 0's by a lane-independent pattern and the row term (a
multiple of the row pitch) to leave the chunk field alone.  This checks it
for every head width, wave count and KV-head count the kernel can be
launched with, against the direct per-lane formula (row * pitch + (chunk ^
swizzle(row)) * 16).  The swizzle is restated here from the kernel's
definition: a 4-bit rotate of the row for rows of 256 bytes or more, a
3-bit pattern for 128-byte rows.
"""
import pytest


def swz(D, r):
    if D >= 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("D", [64, 256, 512])
@pytest.mark.parametrize("waves", [4, 8])
def test_copy_offsets_from_one_register(D, waves):
    row_chunks = D // 8                  # 16-byte chunks per key row
    ops = 32 * row_chunks // 64          # 1 KB copy ops per 32-key tile
    per_wave = -(-ops // waves)
    for hkv in (1, 2, 3, 4, 8, 16):
        pitch = hkv * D * 2
        for wave in range(waves):
            def direct(i, lane):
                pc = (wave * per_wave + i) * 64 + lane
                row = pc // row_chunks
                return row * pitch + ((pc % row_chunks) ^ swz(D, row)) * 16

            r0 = (wave * per_wave * 64) // row_chunks
            for i in range(per_wave):
                if ops % waves and wave * per_wave + i >= ops:
                    break
                ri = ((wave * per_wave + i) * 64) // row_chunks
                dx = (swz(D, ri) ^ swz(D, r0)) << 4
                drow = (ri - r0) * pitch
                for lane in range(64):
                    assert direct(i, lane) == ((direct(0, lane) ^ dx) + drow), (D, waves, hkv, wave, i, lane)
