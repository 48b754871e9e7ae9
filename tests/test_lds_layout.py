"""CPU model of the split kernel's LDS tile layout (the constants and address
formulas of prefix_splitkv.hip, restated): the nine LDS-DMAs of a wave cover
each (key, 16-byte piece) of a 32-key tile exactly once, the QK K-fragment
reads and the PV transposed V reads land on the pieces their MFMA operands
need, and neither read pattern has LDS bank conflicts under the bank model
fitted to the SQ_LDS_BANK_CONFLICT counter (ds_read_b128: 8 lanes of 16 B
per cycle over 32 four-byte banks; ds_read_b64_tr_b16: 32 lanes of 8 B per
cycle over 64 banks)."""

import re
import os

UNIT, GROUP = 9216, 1024
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "speculative_decoding_tree_verify_amd", "csrc", "prefix_splitkv.hip")


def swz(k8):
    return ((k8 & 2) << 1) | ((k8 & 4) >> 1) | (k8 & 1)


def gather_content():
    content = {}
    for c in range(4):
        for lane in range(64):
            for d in range(9):
                addr = c * UNIT + d * GROUP + 16 * lane
                assert addr not in content
                content[addr] = (8 * c + (lane >> 3), 8 * d + ((lane & 7) ^ swz(lane >> 3)))
    return content


def qk_addr(hf, lane, st):
    l16, q4 = lane & 15, lane >> 4
    k8 = l16 & 7
    base = (2 * hf + (l16 >> 3)) * UNIT + k8 * 128 + ((q4 ^ swz(k8)) << 4)
    return (base ^ (64 * (st & 1))) + GROUP * (st >> 1)


def pv_addr(c, lane, hi, f):
    bb, e, s2 = lane >> 4, (lane >> 2) & 3, lane & 3
    kk = e + 4 * hi
    pvb = (bb >> 1) * UNIT + 2 * c * GROUP + kk * 128 + (((2 * (bb & 1) + (s2 >> 1)) ^ swz(kk)) << 4) + 8 * (s2 & 1)
    ks, cb = f >> 2, f & 3
    return (pvb ^ (64 * (cb & 1))) + ks * 2 * UNIT + (cb >> 1) * GROUP


def test_constants_match_the_kernel():
    src = open(SRC).read()
    assert "constexpr int kUnit = 8 * kDqk * 2;" in src and "constexpr int kGroup = 1024;" in src
    assert "return ((k8 & 2) << 1) | ((k8 & 4) >> 1) | (k8 & 1);" in src
    assert re.search(r"constexpr int kM0Step = kGroup - 128;", src)


def test_gathers_cover_each_piece_once():
    content = gather_content()
    assert len(content) == 32 * 72 and len(set(content.values())) == 32 * 72
    assert max(content) + 16 <= 32 * 1152
    for lane in range(64):                 # sources stay inside the 1152-byte row
        for d in range(9):
            assert 16 * ((lane & 7) ^ swz(lane >> 3)) + 128 * d + 16 <= 1152


def test_qk_reads_land_on_their_pieces_without_conflicts():
    content = gather_content()
    for hf in range(2):
        for lane in range(64):
            for st in range(18):
                assert content[qk_addr(hf, lane, st)] == (16 * hf + (lane & 15), 4 * st + (lane >> 4))
        for st in range(18):
            for g in range(8):
                banks = {((qk_addr(hf, lane, st) // 4) + i) % 32 for lane in range(8 * g, 8 * g + 8) for i in range(4)}
                assert len(banks) == 32


def test_pv_reads_land_on_their_columns_without_conflicts():
    content = gather_content()
    for c in range(4):
        for hi in range(2):
            for f in range(8):
                for lane in range(64):
                    addr = pv_addr(c, lane, hi, f)
                    bb, e, s2 = lane >> 4, (lane >> 2) & 3, lane & 3
                    key = 16 * (f >> 2) + 8 * (bb >> 1) + e + 4 * hi
                    col = 128 * c + 32 * (f & 3) + 16 * (bb & 1) + 4 * s2
                    assert content[addr - addr % 16] == (key, col // 8)
                    assert (addr % 16) // 8 == (col % 8) // 4
                for g in range(2):
                    banks = [((pv_addr(c, lane, hi, f) // 4) + i) % 64 for lane in range(32 * g, 32 * g + 32)
                             for i in range(2)]
                    assert len(set(banks)) == 64
