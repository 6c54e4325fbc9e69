"""Bank-conflict model of the gfx950 LDS, measured with a one-wave probe
(each access pattern repeated 4096 times, rocprofv3 SQ_LDS_BANK_CONFLICT /
SQ_INSTS_LDS), used to choose the XOR swizzles of the kernels' LDS tiles.

* 64 banks of 4 bytes.
* A wave's access is served in passes; lanes of different passes never
  conflict:
  - 16-byte reads: four passes of 16 lanes; each half-wave's eight lane
    quads (lanes 4q..4q+3) split by the parity of the bits of q;
  - 8-byte reads and the transposing 8-byte reads: two passes of 32 lanes;
  - 4-byte reads: two passes of 32 lanes over 32 banks (128 bytes);
  - 8-byte writes: four passes of 16 lanes over 32 banks;
  - 16-byte writes: eight passes of 8 lanes over 32 banks.
* Within a pass, a bank holding k distinct dwords costs k - 1 extra
  cycles; the counter reads 0.94 x the sum over passes per instruction.

The model reproduces every one of the 1438 patterns measured (row and
transposed fragment reads, row reads, tile fills and stores under 60
swizzles, lane-pair and address-pair tests).
"""
from __future__ import annotations

SIZE = {"read16": 16, "read8": 8, "read_tr8": 8, "read4": 4, "write8": 8, "write16": 16}


def passes(kind: str):
    if kind == "read16":
        out = []
        for half in (0, 32):
            for par in (0, 1):
                out.append([half + 4 * q + i for q in range(8)
                            if bin(q).count("1") % 2 == par for i in range(4)])
        return out
    if kind in ("read8", "read_tr8", "read4"):
        return [list(range(0, 32)), list(range(32, 64))]
    if kind == "write8":
        return [list(range(s, s + 16)) for s in range(0, 64, 16)]
    if kind == "write16":
        return [list(range(s, s + 8)) for s in range(0, 64, 8)]
    raise ValueError(kind)


def conflict_cycles(kind: str, addrs) -> int:
    """Extra cycles of one wave-wide access (64 byte addresses, None for an
    idle lane): per pass, the largest number of distinct dwords on one bank,
    less one, summed over the passes."""
    nbanks = 32 if kind in ("read4", "write8", "write16") else 64
    total = 0
    for p in passes(kind):
        banks = {}
        for lane in p:
            a = addrs[lane]
            if a is None:
                continue
            for dw in range(a // 4, (a + SIZE[kind]) // 4):
                banks.setdefault(dw % nbanks, set()).add(dw)
        if banks:
            total += max(len(s) for s in banks.values()) - 1
    return total
