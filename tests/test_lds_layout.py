"""Host model of the prefill kernel's LDS tile layout for staging by LDS
loads (pa_prefill.hip, dma_pos and dma_tile; D = 128, 64-key tiles): the
loads fill every slot once with the intended (row, chunk), every operand
read finds what was loaded, K and transposed-V operand reads cover all 64
LDS banks once (4 bytes per bank, 256 bytes per pass of 16 lanes x 16 bytes
or 32 lanes x 8 bytes), each group of 4 load lanes reads one aligned 64-byte
piece of a row, and operand addresses are a per-lane base plus constants."""
import pytest


def pos(r, c):
    """Position (in 2-byte units) of 16-byte chunk c of row r in a tile."""
    b, i = (r >> 2) & 3, r & 3
    return (r >> 4) * 2048 + b * 512 + (16 * (c >> 2) + 4 * i + ((c & 3) ^ b)) * 8


def loaded():
    """(row, chunk) that the loads of wave w, instruction j, lane l put in
    slot l of the 1 KiB at w * 2048 + j * 512."""
    lds = {}
    for w in range(4):
        for j in range(4):
            for l in range(64):
                lds[w * 2048 + j * 512 + l * 8] = (16 * w + 4 * j + ((l >> 2) & 3),
                                                   4 * (l >> 4) + ((l & 3) ^ j))
    return lds


def banks(addr_bytes, nbytes):
    return [((addr_bytes + 4 * k) // 4) % 64 for k in range(nbytes // 4)]


def test_layout_is_a_bijection_matching_the_loads():
    lds = loaded()
    assert len(lds) == 64 * 16
    assert {pos(r, c) for r in range(64) for c in range(16)} == set(lds)
    for r in range(64):
        for c in range(16):
            assert lds[pos(r, c)] == (r, c)


def test_load_quads_read_aligned_64_byte_row_pieces():
    lds = loaded()
    for base in range(0, 8192, 512):
        for q in range(16):
            cells = [lds[base + (4 * q + e) * 8] for e in range(4)]
            assert len({r for r, _ in cells}) == 1
            assert len({c // 4 for _, c in cells}) == 1


@pytest.mark.parametrize("blk", [0, 1])
@pytest.mark.parametrize("kk", range(8))
def test_k_operand_reads(blk, kk):
    # lane: row blk*32 + lane%32, chunk 2kk + lane/32, 16 bytes
    lds = loaded()
    addr = [pos(blk * 32 + (l & 31), 2 * kk + (l >> 5)) for l in range(64)]
    for l in range(64):
        assert lds[addr[l]] == (blk * 32 + (l & 31), 2 * kk + (l >> 5))
    for g in range(4):
        assert len(set(sum((banks(2 * addr[l], 16) for l in range(16 * g, 16 * g + 16)), []))) == 64
    base = [pos(l & 31, 2 * (kk & 1) + (l >> 5)) for l in range(64)]
    assert {a - b for a, b in zip(addr, base)} == {blk * 4096 + (kk >> 1) * 128}


@pytest.mark.parametrize("blk", [0, 1])
@pytest.mark.parametrize("hf", [0, 1])
@pytest.mark.parametrize("mb", range(4))
@pytest.mark.parametrize("second", [0, 8])
def test_v_transposed_reads(blk, hf, mb, second):
    # lane: row blk*32 + hf*16 + (lane/32)*4 + (lane%16)/4 (+8), dims
    # mb*32 + ((lane/16)%2)*16 + 4*(lane%4): 8 bytes
    lds = loaded()
    addr, base = [], []
    for l in range(64):
        src, half = l & 15, l >> 5
        vr = blk * 32 + hf * 16 + half * 4 + (src >> 2) + second
        d0 = mb * 32 + ((l >> 4) & 1) * 16 + 4 * (src & 3)
        a = pos(vr, d0 >> 3) + (d0 & 7)
        assert lds[a - (d0 & 7)] == (vr, d0 >> 3)
        addr.append(a)
        d00 = ((l >> 4) & 1) * 16 + 4 * (src & 3)
        base.append(pos(half * 4 + (src >> 2) + second, d00 >> 3) + (d00 & 7))
    for g in range(2):
        assert len(set(sum((banks(2 * addr[l], 8) for l in range(32 * g, 32 * g + 32)), []))) == 64
    assert {a - b for a, b in zip(addr, base)} == {blk * 4096 + hf * 2048 + mb * 128}
