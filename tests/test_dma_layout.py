"""The LDS layouts of the DMA tile loads (tiled_dma4_body in
paged_kv_varlen_flash_amd/csrc/pagedattn.hip), modelled on the CPU: the index
formulas of its loader and of its operand reads, restated here, must put every
(key row, 16-byte chunk) of a tile in LDS exactly once, give each MFMA operand
read the elements that the row-major layout of attn_tiled_kernel gives it, and
hit all 64 LDS banks once per read.  The kernel runs 32-key tiles; 64-key
tiles (the same formulas over twice the loads) are checked as well."""
import pytest

D = 128
ROW_BYTES_CASES = (256, 1024, 4096)   # Hkv * D * 2 for Hkv = 1, 4, 16
TILE_KEYS = (32, 64)


def loader(row_bytes, kt):
    """{LDS byte offset: (row, chunk)} of the K and V planes of a kt-key tile
    (kt / 4 loads per plane).  Wave w (0..3) issues loads i = w + 4q of each
    plane, q = 0 .. kt / 16 - 1 (16-key group q).  Lane l writes 16 bytes at
    1024 i + 16 l with the chunk its voffset selects."""
    K, V = {}, {}
    for w in range(4):
        rgo, chh = (w >> 1) & 1, w & 1
        for q in range(kt // 16):
            grp, g = q, w + 4 * q
            for l in range(64):
                voff_k = (8 * rgo + (l & 7)) * row_bytes + ((8 * chh + ((l >> 3) ^ rgo)) << 4)
                r8 = l >> 3
                voff_v = (8 * rgo + r8) * row_bytes + ((8 * chh + ((l & 7) ^ (4 * ((r8 >> 1) & 1)))) << 4)
                for voff, M in ((voff_k, K), (voff_v, V)):
                    row_in_grp, rem = divmod(voff, row_bytes)
                    assert rem % 16 == 0 and rem < 2 * D and row_in_grp < 16
                    dst = 1024 * g + 16 * l
                    assert 0 <= dst < kt * 2 * D and dst not in M
                    M[dst] = (16 * grp + row_in_grp, rem // 16)
    return K, V


def k_read(lane, t, u):
    n, h = lane & 31, lane >> 5
    n8 = n >> 3
    return 2048 * n8 + 128 * (h ^ (n8 & 1)) + 16 * (n & 7) + 8192 * u + 1024 * (t >> 2) + 256 * (t & 3)


def v_read(lane, dt, ks, e):
    h, q16, s16 = lane >> 5, lane >> 4, lane & 15
    r8 = 4 * h + (s16 >> 2)
    cl = 2 * (q16 & 1) + ((s16 & 3) >> 1)
    vb0 = 128 * r8 + 16 * cl + 8 * (s16 & 1) + 64 * ((r8 >> 1) & 1)
    return (vb0 ^ 64 if dt & 1 else vb0) + 4096 * ks + 2048 * e + 1024 * (dt >> 1)


@pytest.mark.parametrize("kt", TILE_KEYS)
@pytest.mark.parametrize("row_bytes", ROW_BYTES_CASES)
def test_every_chunk_once(row_bytes, kt):
    K, V = loader(row_bytes, kt)
    full = sorted((r, c) for r in range(kt) for c in range(16))
    assert sorted(K.values()) == full and sorted(V.values()) == full


@pytest.mark.parametrize("kt", TILE_KEYS)
@pytest.mark.parametrize("row_bytes", ROW_BYTES_CASES)
def test_operand_reads_match_row_major(row_bytes, kt):
    K, V = loader(row_bytes, kt)
    for lane in range(64):
        n, h = lane & 31, lane >> 5
        q16, s16 = lane >> 4, lane & 15
        for t in range(8):
            for u in range(kt // 32):
                # K operand of k-step t, key half u: row n + 32u, d 16t + 8h .. +7
                assert K[k_read(lane, t, u)] == (n + 32 * u, 2 * t + h)
        for dt in range(4):
            for ks in range(kt // 16):
                for e in range(2):
                    # transposing read: 8 bytes of row 16ks + 8e + 4h + s16/4
                    # at element 32dt + 16(q16 % 2) + 4(s16 % 4)
                    unit, half = divmod(v_read(lane, dt, ks, e), 16)
                    row, chunk = V[16 * unit]
                    assert row == 16 * ks + 8 * e + 4 * h + (s16 >> 2)
                    assert 16 * chunk + half == 2 * (32 * dt + 16 * (q16 & 1) + 4 * (s16 & 3))


def test_reads_hit_every_bank_once():
    for t in range(8):
        for u in range(2):
            for g0 in range(0, 64, 16):       # 16 lanes x 16 bytes per cycle
                banks = {(k_read(l, t, u) // 4 + w) % 64 for l in range(g0, g0 + 16) for w in range(4)}
                assert len(banks) == 64
    for dt in range(4):
        for ks in range(4):
            for e in range(2):
                for g0 in (0, 32):            # 32 lanes x 8 bytes per cycle
                    banks = {(v_read(l, dt, ks, e) // 4 + w) % 64
                             for l in range(g0, g0 + 32) for w in range(2)}
                    assert len(banks) == 64


def test_staged_epilogue_fits_both_slots():
    """The staged output of 4 waves (8 KB each) goes to both slots of both
    planes of a 32-key-tile workgroup: waves 0-1 in the K slots, 2-3 in the V
    slots, 8 KB apart."""
    slot_bytes = 32 * 2 * D
    for w in range(4):
        off = 8192 * (w & 1)
        assert off + 8192 <= 2 * slot_bytes
