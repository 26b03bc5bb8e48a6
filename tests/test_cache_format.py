"""The tests' statement of the cache byte format (tests/cache_format.py), checked on its own.

The format module is what the GPU tests read device blobs with, so it is pinned here by
things other than itself: packed words derived by hand from its specification, the
packing golden words, byte round trips in both directions, and the structure of the value
stream order. It imports nothing from the oracle or the library.
"""
import dataclasses
import os

import numpy as np
import pytest

from tests import cache_format as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@dataclasses.dataclass
class Cfg:
    batch: int
    n_kv: int
    head_dim: int
    capacity: int
    n_sink: int
    n_recent: int
    quant: str
    k_bits: tuple
    v_bits: tuple
    key_norm: bool = False


def _rand_content(rng, cfg, h, T):
    D = cfg.head_dim
    Gd = D // 32
    ns = min(T, cfg.n_sink)
    body = F.body_tokens(T, cfg.n_sink, cfg.n_recent)
    nblk = body // 32
    kb, vb = cfg.k_bits[h], cfg.v_bits[h]
    hyb = cfg.quant == "hybrid"
    f16 = lambda shape: rng.integers(0, 1 << 16, size=shape, dtype=np.uint16).view(np.float16)
    c = {}
    if kb == 16:
        c["k_raw"] = rng.integers(0, 1 << 16, size=(body, D), dtype=np.uint16)
    else:
        c["k_codes"] = rng.integers(0, 1 << kb, size=(body, Gd, 32)).astype(np.uint8)
        c["k_s"], c["k_z"] = f16((body, Gd)), f16((body, Gd))
        c["k_flag"] = (rng.integers(0, 2, size=(body, Gd)) * hyb).astype(np.uint8)
    if vb == 16:
        c["v_raw"] = rng.integers(0, 1 << 16, size=(body, D), dtype=np.uint16)
    else:
        c["v_codes"] = rng.integers(0, 1 << vb, size=(nblk, D, 32)).astype(np.uint8)
        c["v_s"], c["v_z"] = f16((nblk, D)), f16((nblk, D))
        c["v_flag"] = (rng.integers(0, 2, size=(nblk, D)) * hyb).astype(np.uint8)
    for key, n in (("sink_k", ns), ("sink_v", ns), ("win_k", T - ns - body), ("win_v", T - ns - body)):
        c[key] = rng.integers(0, 1 << 16, size=(n, D), dtype=np.uint16)
    if cfg.key_norm and kb != 16:
        c["k_norm"] = (2.0 ** rng.integers(-3, 4, size=D)).astype(np.float32)
    return c


CASES = [
    Cfg(1, 7, 128, 1000, 4, 128, "hybrid", (2, 3, 4, 5, 6, 7, 8), (8, 7, 6, 5, 4, 3, 2), key_norm=True),
    Cfg(1, 4, 64, 700, 1, 32, "asym", (16, 3, 2, 16), (2, 16, 5, 16)),
    Cfg(1, 3, 128, 300, 0, 0, "hybrid", (16, 4, 3), (3, 16, 2)),
]


@pytest.mark.parametrize("cfg", CASES, ids=["hybrid-all-widths", "asym-16bit-sides", "no-windows"])
@pytest.mark.parametrize("T", [0, 1, 5, 163, 195, 290, 291])
def test_decode_of_encode_is_identity(cfg, T):
    rng = np.random.default_rng(1000 + T)
    T = min(T, cfg.capacity)
    for h in range(cfg.n_kv):
        want = _rand_content(rng, cfg, h, T)
        data, mask = F.encode_head(want, cfg, h, T)
        assert [d.size for d in data] == F.region_sizes(cfg, h)
        got = F.decode_head(data, cfg, h, T)
        F.assert_content_equal(got, want, f"head {h} T {T}")


@pytest.mark.parametrize("cfg", CASES[:2], ids=["hybrid-all-widths", "asym-16bit-sides"])
def test_encode_of_decode_restores_defined_bytes(cfg):
    rng = np.random.default_rng(7)
    T = cfg.capacity - 3
    for h in range(cfg.n_kv):
        regions = [rng.integers(0, 256, size=s, dtype=np.uint8) for s in F.region_sizes(cfg, h)]
        data, mask = F.encode_head(F.decode_head(regions, cfg, h, T), cfg, h, T)
        for r in range(F.N_REGIONS):
            assert np.array_equal(data[r][mask[r]], regions[r][mask[r]]), (h, r)
        # every byte of a full body's code and meta regions is defined (no gaps in the format)
        kb, vb = cfg.k_bits[h], cfg.v_bits[h]
        body = F.body_tokens(T, cfg.n_sink, cfg.n_recent)
        if kb != 16 and body % 64 == 0:
            assert mask[F.KC].all() and mask[F.KM].all(), h
        if vb != 16 and body % 64 == 0:
            assert mask[F.VC].all() and mask[F.VM].all(), h


def test_pack_stream_golden_words():
    for line in open(os.path.join(GOLDEN, "pack_words.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        b = int(parts[0])
        want = np.array([int(x, 16) for x in parts[1:]], dtype=np.uint32)
        codes = np.arange(32) % (1 << b)
        assert np.array_equal(F.pack_stream(codes, b), want), b
        assert np.array_equal(F.unpack_stream(want, b), codes), b


def test_hand_derived_words():
    """Word positions worked out by hand from the specification text."""
    # keys, D 128, 3 bits: W = 12. Token 65 is token 1 of tile 1; its word 5 is word 2 of group 1
    # and lies in chunk q = 1 (nq = 4): uint32 1 * 64 * 12 + 256 + 1 * 4 + 1 = 1029. With group 1
    # holding codes i mod 8, its words are the 3-bit golden words, word 2 = 0xFAC688FA.
    cfg = Cfg(1, 1, 128, 400, 4, 128, "hybrid", (3,), (2,))
    T = 4 + 128 + 128  # body 128: tiles 0 and 1, blocks 0..3
    c = _rand_content(np.random.default_rng(3), cfg, 0, T)
    c["k_codes"][65, 1] = np.arange(32) % 8
    # values, 2 bits: block 3 = half 1 of tile 1. Channel 53 = 16 * 3 + 5 (n 5, nb 3) and channel
    # 37 = 16 * 2 + 5 share stream vg 1 of lane records n = 5; jp = 1 is lane 16 (2 + 1) + 5 = 53,
    # whose stream 1 starts at uint32 (64 + 53) * 4 * 2 + 2 = 938. Elements 0..15 (chunks 0, 1:
    # channel 37) sit at stream positions 0..15 (word 0), elements 16..31 (channel 53) at
    # positions 16..31 (word 1). Tokens of jp = 1 are 8..15 and 24..31 of the block.
    jp1 = np.r_[8:16, 24:32]
    c["v_codes"][3, :, :] = 0
    c["v_codes"][3, 37, jp1] = 1
    c["v_codes"][3, 53, jp1] = 2
    c["v_s"][3, 53] = np.float16(1.0)
    c["v_z"][3, 53] = np.float16(-2.0)
    c["k_flag"][:] = 0
    c["v_flag"][:] = 0
    c["k_flag"][3 * 32 + 5, 2] = 1  # token 5 of block 3, group 2: key flag bit 5 * 4 + 2 = 22
    c["v_flag"][3, 53] = 1           # value flag bit 53: word 1, bit 21
    data, _ = F.encode_head(c, cfg, 0, T)
    kc, vc, vm, fl = (data[r].view(np.uint32) for r in (F.KC, F.VC, F.VM, F.FL))
    assert kc[1029] == 0xFAC688FA
    assert vc[938] == 0x55555555 and vc[939] == 0xAAAAAAAA
    # value meta of block 3, channel 53: uint32 1 * 256 + 1 * 128 + 5 * 8 + 3 = 427, s | z << 16
    assert vm[427] == 0xC0003C00
    # flags of block 3: key words 24..27, value words 28..31
    assert fl[24] == 1 << 22 and fl[25] == 0 and fl[28] == 0 and fl[29] == 1 << 21
    # keys with W mod 4 = 2 (D 64, 3 bits, W = 6): token 10 of tile 0, words 4 and 5 (group 1,
    # words 1 and 2) are chunk 1 with nq = 2: uint32 256 + 10 * 2 + 0 and + 1
    cfg2 = Cfg(1, 1, 64, 300, 0, 32, "asym", (3,), (3,))
    c2 = _rand_content(np.random.default_rng(4), cfg2, 0, 100)
    c2["k_codes"][10, 1] = np.arange(32) % 8
    kc2 = F.encode_head(c2, cfg2, 0, 100)[0][F.KC].view(np.uint32)
    assert kc2[276] == 0xC688FAC6 and kc2[277] == 0xFAC688FA
    # ring: n_sink 4, n_recent 128 -> 160 slots; token 300 sits in slot (300 - 4) mod 160 = 136
    cfg3 = Cfg(1, 1, 64, 400, 4, 128, "asym", (2,), (2,))
    c3 = _rand_content(np.random.default_rng(5), cfg3, 0, 301)
    rk = F.encode_head(c3, cfg3, 0, 301)[0][F.RK].view(np.uint16).reshape(160, 64)
    assert np.array_equal(rk[136], c3["win_k"][300 - 4 - F.body_tokens(301, 4, 128)])


def test_value_stream_order_is_a_permutation_one_window_per_register():
    # every width's order covers positions 0..31 once; the decode kernel reads the two codes of
    # a register (elements 4 r + 2 h, 4 r + 2 h + 1 of a chunk's step) with one shift and one
    # mask, so their fields, read from one 32-bit window, must sit in the low and high 16-bit
    # halves at most 10 - b bits up
    for b in range(2, 9):
        pos = F.VALUE_STREAM_POS[b]
        assert sorted(pos) == list(range(32)), b
        for e in range(0, 32, 2):
            lo, hi = pos[e], pos[e + 1]
            gap = b * (hi - lo) - 16
            assert abs(gap) <= 10 - b, (b, e, lo, hi)
