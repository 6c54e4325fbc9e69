"""The LDS tile layouts against the measured gfx950 bank model
(recurrent_attention_amd/lds_banks.py): every fragment read of the
kernels' row-major and transposed tiles, and their fills, are free of bank
conflicts under the swizzles the kernels use, where the earlier swizzles
left the listed patterns two-way conflicted.  The 8-byte stores of
matrix-core outputs (16 lanes writing one half-unit column of 16 rows) are
two-way under any XOR swizzle; the test pins that too, so that a claim of
more is caught."""
import pytest

from recurrent_attention_amd.lds_banks import conflict_cycles

LANES = range(64)


# ---- the swizzles of the kernels (unit XOR as a function of the row)
def bf16_256(row):          # 256-byte bf16 rows (tile_ops.h bw_swz, mask 15)
    return (row ^ ((row & 1) * 12)) & 15


def bf16_256_old(row):
    return row & 15


def tr_128(row):            # 128-byte transposed tiles (chunk_kernel.h tr_pos)
    return (row ^ (row >> 2)) & 7


def tr_128_old(row):
    return (row ^ (row >> 3)) & 7


def cc_128(row):            # 64 x 64 bf16 P and T tiles of the delta rule (delta_kernel.h cc_pos)
    return (row ^ (row >> 3)) & 7


def cc_128_old(row):
    return row & 7


def g_512(row):             # fp32 G tile of the gradient kernel (bwd_kernel.h g_pos)
    return (row & 3) | ((((row >> 2) ^ (row >> 3)) & 1) << 2) | (((row >> 2) & 1) << 3)


def g_512_old(row):
    return (row ^ (row >> 4)) & 15


def bf16_addr(f, row_bytes):
    def a(row, col):        # bf16 column -> byte address, 16-byte units
        return row * row_bytes + ((col // 8) ^ f(row)) * 16 + (col % 8) * 2
    return a


def pats_256(a):
    """Access patterns on a [64][128] bf16 tile (rows of 256 bytes)."""
    rowfrag = [conflict_cycles("read16", [a(16 * tb + (l & 15), 32 * kk + 8 * (l >> 4)) for l in LANES])
               for tb in range(4) for kk in range(4)]
    tr = [conflict_cycles("read_tr8", [a(k0 + 8 * (l >> 4) + ((l & 15) >> 2) + ex, c0 + 4 * (l & 3))
                                       for l in LANES])
          for k0 in (0, 32) for c0 in range(0, 128, 16) for ex in (0, 4)]
    rowread = [conflict_cycles("read8", [a(16 * xb + (l & 15), 32 * k2 + off + 4 * (l >> 4)) for l in LANES])
               for xb in range(4) for k2 in range(4) for off in (0, 16)]
    fill = [conflict_cycles("write8", [a((l >> 5) + 2 * w + 16 * ps, 4 * (l & 31)) for l in LANES])
            for w in range(8) for ps in range(4)]
    out8 = [conflict_cycles("write8", [a(16 * sb + (l & 15), n0 + 4 * (l >> 4)) for l in LANES])
            for sb in range(4) for n0 in range(0, 128, 16)]
    return {k: max(v) for k, v in dict(rowfrag=rowfrag, tr=tr, rowread=rowread, fill=fill,
                                       out8=out8).items()}


def test_256_byte_rows():
    new = pats_256(bf16_addr(bf16_256, 256))
    old = pats_256(bf16_addr(bf16_256_old, 256))
    assert new == {"rowfrag": 0, "tr": 0, "rowread": 0, "fill": 0, "out8": 4}
    assert old["tr"] == 2 and old["rowfrag"] == 0


def test_256_byte_rows_token_pairs_16_apart():
    """The delta rule's transposing reads of K and V (rows 4 g + i and
    16 + 4 g + i of a 32-token group, matching a matrix-core result used as
    the next operand) stay conflict-free under the same swizzle."""
    a = bf16_addr(bf16_256, 256)
    tr = [conflict_cycles("read_tr8", [a(k0 + 4 * (l >> 4) + ((l & 15) >> 2) + ex, c0 + 4 * (l & 3))
                                       for l in LANES])
          for k0 in (0, 32) for c0 in range(0, 128, 16) for ex in (0, 16)]
    assert max(tr) == 0


def test_delta_64_by_64_tiles():
    """P and T, [64][64] bf16 (rows of 128 bytes), read in 8-byte row reads
    (rows 16 b + r, columns 32 k + 4 g and 32 k + 16 + 4 g)."""
    def rowread(f):
        a = bf16_addr(f, 128)
        return max(conflict_cycles("read8", [a(16 * xb + (l & 15), 32 * k2 + off + 4 * (l >> 4)) for l in LANES])
                   for xb in range(4) for k2 in range(2) for off in (0, 16))
    assert rowread(cc_128) == 0
    assert rowread(cc_128_old) == 2


def pats_tr128(a):
    """The transposed K / V tiles of the chunk kernels: [128][64] bf16."""
    frag = [conflict_cycles("read16", [a(16 * mb + (l & 15), 32 * kk + 8 * (l >> 4)) for l in LANES])
            for mb in range(8) for kk in range(2)]
    # fill: lane l holds 4 channels (rows 4 (l % 32) + i) of 4 tokens
    store = [conflict_cycles("write8", [a(4 * (l % 32) + i, 8 * w + 4 * (l // 32)) for l in LANES])
             for w in range(8) for i in range(4)]
    return max(frag), max(store)


def test_transposed_128_byte_rows():
    assert pats_tr128(bf16_addr(tr_128, 128)) == (0, 4)
    assert pats_tr128(bf16_addr(tr_128_old, 128)) == (4, 4)


def g_addr(f):
    def a(row, col):        # fp32 [128][128], 16-byte units
        return 4 * (row * 128 + ((((col >> 2) ^ f(row)) << 2) | (col & 3)))
    return a


def pats_g(a):
    col = [conflict_cycles("read4", [a(kk * 32 + 8 * (l >> 4) + j, 16 * nb + (l & 15)) for l in LANES])
           for kk in range(4) for j in range(8) for nb in range(8)]
    upd = [conflict_cycles(k, [a(16 * x + (l & 15), 16 * c + 4 * (l >> 4)) for l in LANES])
           for x in range(8) for c in range(8) for k in ("read16", "write16")]
    rows = [conflict_cycles("read16", [a(16 * nb + (l & 15), kk * 32 + 8 * (l >> 4) + off) for l in LANES])
            for nb in range(8) for kk in range(4) for off in (0, 4)]
    return max(col), max(upd), max(rows)


def test_g_tile():
    assert pats_g(g_addr(g_512)) == (0, 0, 0)
    assert pats_g(g_addr(g_512_old))[0] == 2


@pytest.mark.parametrize("f,units", [(bf16_256, 16), (tr_128, 8), (cc_128, 8), (g_512, 32)])
def test_swizzles_keep_each_row_a_permutation(f, units):
    for row in range(128):
        assert sorted(u ^ f(row) for u in range(units)) == list(range(units))
