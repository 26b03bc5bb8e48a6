"""Byte format of a libkvq cache blob, as the tests read it.

The pages define no storage format: this is the library's own. It is written here from its
specification, which this docstring states in full. The module is independent of the CPU
oracle, which holds only the logical content of a cache (codes, scales, zeros, flags, 16-bit
rows and norms), and of the kernels' unpack code. The GPU tests decode a device blob with
``decode_head`` and compare the logical content with the oracle's bit for bit; the decode
kernel reading the same bytes is checked by its attention output. ``encode_head`` is the
inverse, used to test this module on its own (byte round trips, hand-derived words).

Specification
-------------
Blob: a 256-byte header, then the region table ``uint64 off[B][Hkv][10]`` at byte 256, then
the regions in (row, KV head, region) order, each starting on a 256-byte boundary. The ten
regions of one (row, KV head) are KC, KM, VC, VM, FL, SK, SV, RK, RV, KN.

Geometry: bmax = 32 * max(0, (capacity - n_sink - n_recent) // 32) body tokens at most,
nblk = bmax / 32 value blocks, ntile = ceil(nblk / 2) tiles of 64 tokens, Gd = D / 32 groups
per token. A group's 32 b-bit codes form a little-endian bitstream of b uint32 words: code i
occupies stream bits [i b, i b + b), and stream bit k is bit k mod 32 of word k div 32.
(s, z) pairs are stored as one uint32 word, s | z << 16 (float16 bit patterns).

KC  key codes, ntile * 64 * D * kb / 8 bytes. Token t of the body (tile t div 64, tt = t mod
    64) has W = Gd * kb words, group g's bitstream at words g * kb .. g * kb + kb - 1. The
    words are cut into 16-byte chunks q = w div 4 (the last one 8 bytes when W mod 4 = 2);
    chunk q of the tile's 64 tokens is stored contiguously, so word w of token tt is uint32
    tile * 64 * W + 256 q + tt * nq + (w - 4 q), nq = min(4, W - 4 q).
KM  key (s, z), ntile * 64 * Gd words: word t * Gd + g.
VC  value codes, ntile * 64 * D * vb / 8 bytes. Value block j (body tokens 32 j .. 32 j + 31)
    is half blk = j mod 2 of tile j div 2. A tile holds 64 lane records l = 16 (2 blk + jp) +
    n (jp = 0, 1; n = 0..15) of Gd streams of vb words; stream vg of record l starts at
    uint32 (tile * 64 + l) * Gd * vb + vg * vb. Its element e = 8 c + u (chunk c = 0..3, u =
    0..7) is the code of channel 16 (2 vg + c div 2) + n and token 16 (c mod 2) + 8 jp + u of
    block j, and it sits at position VALUE_STREAM_POS[vb][e] of the stream, which is packed
    as a group's bitstream.
VM  value (s, z), ntile * 2 * D words: block j, channel c = 16 nb + n at word
    (j div 2) * 2 D + (j mod 2) * D + n * (D / 16) + nb.
FL  hybrid flags (hybrid caches only), nblk * 2 * Gd words. Block j's key flags are a
    bitstream of Gd words at word j * 2 Gd, flag of (token tt of the block, group g) at bit
    tt * Gd + g; its value flags follow at word j * 2 Gd + Gd, flag of channel c at bit c.
    A flag of 1 marks the symmetric variant. The flags of a 16-bit side are not written.
SK  sink keys, n_sink * D 16-bit values, row u at [u][D]; SV the same for values.
RK  recent-ring keys, (n_recent + 32) * D 16-bit values; token t >= n_sink at slot
    (t - n_sink) mod (n_recent + 32); RV the same for values.
KN  per-channel key norms, D float32 (key normalization on a quantized key head, else empty).

A head with 16-bit keys stores KC as bmax rows [t][D] of the input dtype, and KM is empty;
likewise VC and VM for 16-bit values.

Paged caches: KC..FL of each head are pools of pages, one page per 64-token tile, a page's
bytes laid out as that tile's bytes in a contiguous cache (KC 64 W * 4, KM 64 Gd * 4, VC
8 D vb, VM 8 D, FL 16 Gd; 16-bit sides 64 * 2 D).
"""
from __future__ import annotations

import numpy as np

HEADER_BYTES = 256
N_REGIONS = 10
KC, KM, VC, VM, FL, SK, SV, RK, RV, KN = range(N_REGIONS)
TILE = 64
GROUP = 32

# Position, inside a 32-code value stream of width b, of element e = 8 c + u (chunk c, token
# u of the chunk). The order is chosen so that pairs of codes that the decode kernel separates
# with one shift and one mask sit at fixed distances in the stream.
VALUE_STREAM_POS = {
    2: [0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15, 16, 24, 17, 25, 18, 26, 19, 27, 20, 28, 21, 29, 22, 30,
        23, 31],
    3: [0, 5, 1, 6, 2, 7, 10, 15, 11, 16, 20, 26, 21, 27, 24, 30, 3, 8, 4, 9, 14, 19, 12, 17, 13, 18, 22, 28, 23, 29,
        25, 31],
    4: [0, 4, 1, 5, 2, 6, 3, 7, 8, 12, 9, 13, 10, 14, 11, 15, 16, 20, 17, 21, 18, 22, 19, 23, 24, 28, 25, 29, 26, 30,
        27, 31],
    5: [0, 3, 2, 5, 7, 10, 8, 12, 15, 18, 20, 23, 22, 25, 27, 30, 1, 4, 6, 9, 11, 14, 13, 17, 16, 19, 21, 24, 26, 29,
        28, 31],
    6: [0, 3, 1, 4, 6, 8, 7, 10, 11, 14, 15, 18, 21, 24, 26, 29, 28, 31, 2, 5, 17, 19, 9, 12, 13, 16, 20, 23, 22, 25,
        27, 30],
    7: [0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30, 1, 3, 5, 7, 9, 11, 13, 15, 17, 19, 21, 23, 25, 27,
        29, 31],
    8: [0, 2, 1, 3, 4, 6, 5, 7, 8, 10, 9, 11, 12, 14, 13, 15, 16, 18, 17, 19, 20, 22, 21, 23, 24, 26, 25, 27, 28, 30,
        29, 31],
}


def body_tokens(T: int, n_sink: int, n_recent: int) -> int:
    """Quantized body after T tokens: whole 32-token blocks past the sink and the window."""
    return GROUP * max(0, (T - n_sink - n_recent) // GROUP)


def ring_slots(n_recent: int) -> int:
    return n_recent + GROUP


def _align(x, a=256):
    return (x + a - 1) // a * a


def region_sizes(cfg, h):
    """Bytes of the ten regions of one (row, KV head) of cache config `cfg` (fields batch,
    n_kv, head_dim, capacity, n_sink, n_recent, quant, k_bits, v_bits, key_norm)."""
    D = cfg.head_dim
    bmax = body_tokens(cfg.capacity, cfg.n_sink, cfg.n_recent)
    nblk = bmax // GROUP
    ntile = (nblk + 1) // 2
    kb, vb = cfg.k_bits[h], cfg.v_bits[h]
    sz = [0] * N_REGIONS
    sz[KC] = bmax * D * 2 if kb == 16 else ntile * TILE * D * kb // 8
    sz[KM] = 0 if kb == 16 else ntile * TILE * (D // GROUP) * 4
    sz[VC] = bmax * D * 2 if vb == 16 else ntile * TILE * D * vb // 8
    sz[VM] = 0 if vb == 16 else ntile * 2 * D * 4
    sz[FL] = nblk * 2 * (D // GROUP) * 4 if cfg.quant == "hybrid" else 0
    sz[SK] = sz[SV] = cfg.n_sink * D * 2
    sz[RK] = sz[RV] = ring_slots(cfg.n_recent) * D * 2
    sz[KN] = D * 4 if cfg.key_norm and kb != 16 else 0
    return sz


def tile_bytes(cfg, h):
    """Bytes of one 64-token tile of regions KC..FL of head h: the page sizes of its pools."""
    D, kb, vb = cfg.head_dim, cfg.k_bits[h], cfg.v_bits[h]
    return [TILE * D * 2 if kb == 16 else TILE * D * kb // 8,
            0 if kb == 16 else TILE * (D // GROUP) * 4,
            TILE * D * 2 if vb == 16 else TILE * D * vb // 8,
            0 if vb == 16 else 2 * D * 4,
            2 * 2 * (D // GROUP) * 4 if cfg.quant == "hybrid" else 0]


def layout(cfg):
    """Region offsets (bytes from the blob start) [B][H][10] and the blob size."""
    B, H = cfg.batch, cfg.n_kv
    off = np.zeros((B, H, N_REGIONS), dtype=np.uint64)
    pos = _align(HEADER_BYTES + B * H * N_REGIONS * 8)
    for b in range(B):
        for h in range(H):
            sz = region_sizes(cfg, h)
            for r in range(N_REGIONS):
                off[b, h, r] = pos
                pos = _align(pos + sz[r])
    return off, pos


# ------------------------------------------------------------------------- bitstreams ------

def pack_stream(codes: np.ndarray, b: int) -> np.ndarray:
    """[..., 32] codes of b bits -> [..., b] uint32 words (little-endian bitstream)."""
    codes = np.asarray(codes, dtype=np.uint64)
    bits = (codes[..., :, None] >> np.arange(b, dtype=np.uint64)) & np.uint64(1)   # [..., i, j]: stream bit i b + j
    bits = bits.reshape(codes.shape[:-1] + (b, 32))                                 # [..., word, bit]
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def unpack_stream(words: np.ndarray, b: int) -> np.ndarray:
    """[..., b] uint32 words -> [..., 32] codes (inverse of pack_stream)."""
    words = np.asarray(words, dtype=np.uint64)
    bits = (words[..., :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)   # [..., word, bit]
    bits = bits.reshape(words.shape[:-1] + (32, b))                                 # [..., i, j]
    return (bits << np.arange(b, dtype=np.uint64)).sum(axis=-1).astype(np.uint8)


def _bits_to_words(flags: np.ndarray) -> np.ndarray:
    """[..., 32 n] 0/1 flags -> [..., n] uint32 (bit i at word i div 32, bit i mod 32)."""
    f = np.asarray(flags, dtype=np.uint64)
    f = f.reshape(f.shape[:-1] + (f.shape[-1] // 32, 32))
    return (f << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


def _words_to_bits(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words, dtype=np.uint64)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,)).astype(np.uint8)


# ------------------------------------------------------------------------- index maps -----

def key_word_index(body: int, W: int) -> np.ndarray:
    """uint32 index in KC of word w of body token t, as an int64 array [body][W]."""
    t = np.arange(body)[:, None]
    w = np.arange(W)[None, :]
    q = w // 4
    nq = np.minimum(4, W - 4 * q)
    return (t // TILE) * (TILE * W) + 256 * q + (t % TILE) * nq + (w - 4 * q)


def value_maps(nblk: int, D: int, vb: int):
    """For every value code (block j, channel c, token i of the block): the uint32 index of the
    first word of its stream in VC and its position in that stream; arrays [nblk][D][32]."""
    Gd = D // GROUP
    j = np.arange(nblk)[:, None, None]
    c = np.arange(D)[None, :, None]
    i = np.arange(GROUP)[None, None, :]
    n, nb = c % 16, c // 16
    vg, chunk_hi = nb // 2, nb % 2                # stream, chunk c div 2
    kk, jp, u = i // 16, (i // 8) % 2, i % 8     # token i = 16 kk + 8 jp + u
    e = 8 * (2 * chunk_hi + kk) + u
    lane = 16 * (2 * (j % 2) + jp) + n
    word0 = ((j // 2) * TILE + lane) * Gd * vb + vg * vb
    pos = np.asarray(VALUE_STREAM_POS[vb])[e]
    return np.broadcast_to(word0, (nblk, D, GROUP)), np.broadcast_to(pos, (nblk, D, GROUP))


def value_meta_index(nblk: int, D: int) -> np.ndarray:
    """uint32 index in VM of (block j, channel c), [nblk][D]."""
    j = np.arange(nblk)[:, None]
    c = np.arange(D)[None, :]
    return (j // 2) * 2 * D + (j % 2) * D + (c % 16) * (D // 16) + c // 16


# ------------------------------------------------------------------------- decode ---------

def _u32(region: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(region).view(np.uint32)


def _u16(region: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(region).view(np.uint16)


def _meta(words: np.ndarray):
    s = (words & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16)
    z = (words >> np.uint32(16)).astype(np.uint16).view(np.float16)
    return s, z


def decode_head(regions, cfg, h: int, T: int) -> dict:
    """Logical content of one (row, KV head) holding T tokens, read from its ten regions
    (uint8 arrays). Keys of the result, shaped like the oracle's cache fields of one row:
    k_codes [body][Gd][32], k_s, k_z, k_flag [body][Gd] (or k_raw [body][D] for 16-bit keys),
    v_codes [nblk][D][32], v_s, v_z, v_flag [nblk][D] (or v_raw), sink_k, sink_v [ns][D],
    win_k, win_v [T - ns - body][D] in token order, and k_norm [D] when stored."""
    D = cfg.head_dim
    Gd = D // GROUP
    kb, vb = cfg.k_bits[h], cfg.v_bits[h]
    ns = min(T, cfg.n_sink)
    body = body_tokens(T, cfg.n_sink, cfg.n_recent)
    nblk = body // GROUP
    hyb = cfg.quant == "hybrid"
    out = {}
    if kb == 16:
        out["k_raw"] = _u16(regions[KC])[:body * D].reshape(body, D).copy()
    else:
        W = Gd * kb
        words = _u32(regions[KC])[key_word_index(body, W)]                       # [body][W]
        out["k_codes"] = unpack_stream(words.reshape(body, Gd, kb), kb)
        out["k_s"], out["k_z"] = _meta(_u32(regions[KM])[:body * Gd].reshape(body, Gd))
        if hyb:
            fw = _u32(regions[FL]).reshape(-1, 2 * Gd)[:nblk, :Gd]                # [nblk][Gd]
            out["k_flag"] = _words_to_bits(fw).reshape(nblk, GROUP, Gd).reshape(body, Gd)
        else:
            out["k_flag"] = np.zeros((body, Gd), dtype=np.uint8)
    if vb == 16:
        out["v_raw"] = _u16(regions[VC])[:body * D].reshape(body, D).copy()
    else:
        word0, pos = value_maps(nblk, D, vb)
        vc = _u32(regions[VC])
        streams = vc[word0[..., None] + np.arange(vb)]                              # [nblk][D][32][vb]
        codes = unpack_stream(streams, vb)                                          # [nblk][D][32][32]
        out["v_codes"] = np.take_along_axis(codes, pos[..., None], axis=-1)[..., 0]
        out["v_s"], out["v_z"] = _meta(_u32(regions[VM])[value_meta_index(nblk, D)])
        if hyb:
            fw = _u32(regions[FL]).reshape(-1, 2 * Gd)[:nblk, Gd:]
            out["v_flag"] = _words_to_bits(fw)
        else:
            out["v_flag"] = np.zeros((nblk, D), dtype=np.uint8)
    out["sink_k"] = _u16(regions[SK])[:ns * D].reshape(ns, D).copy()
    out["sink_v"] = _u16(regions[SV])[:ns * D].reshape(ns, D).copy()
    R = ring_slots(cfg.n_recent)
    toks = np.arange(ns + body, T)
    slots = (toks - cfg.n_sink) % R
    out["win_k"] = _u16(regions[RK]).reshape(R, D)[slots].copy()
    out["win_v"] = _u16(regions[RV]).reshape(R, D)[slots].copy()
    if regions[KN].size:
        out["k_norm"] = np.ascontiguousarray(regions[KN]).view(np.float32).copy()
    return out


# ------------------------------------------------------------------------- encode ---------

def encode_head(content: dict, cfg, h: int, T: int):
    """Inverse of decode_head: the ten regions (uint8 arrays) of one (row, KV head) from its
    logical content, and a mask per region of the bytes that content defines."""
    D = cfg.head_dim
    Gd = D // GROUP
    kb, vb = cfg.k_bits[h], cfg.v_bits[h]
    ns = min(T, cfg.n_sink)
    body = body_tokens(T, cfg.n_sink, cfg.n_recent)
    nblk = body // GROUP
    sz = region_sizes(cfg, h)
    data = [np.zeros(s, dtype=np.uint8) for s in sz]
    mask = [np.zeros(s, dtype=bool) for s in sz]

    def put32(r, idx, vals):
        w = data[r].view(np.uint32)
        w[idx.reshape(-1)] = np.asarray(vals, dtype=np.uint32).reshape(-1)
        m = mask[r].reshape(-1, 4)
        m[idx.reshape(-1)] = True

    def put16(r, rows):
        raw = np.ascontiguousarray(rows, dtype=np.uint16).reshape(-1).view(np.uint8)
        data[r][:raw.size] = raw
        mask[r][:raw.size] = True

    if kb == 16:
        put16(KC, content["k_raw"])
    elif body:
        W = Gd * kb
        words = pack_stream(content["k_codes"], kb).reshape(body, W)
        put32(KC, key_word_index(body, W), words)
        meta = (content["k_s"].view(np.uint16).astype(np.uint32)
                | (content["k_z"].view(np.uint16).astype(np.uint32) << np.uint32(16)))
        put32(KM, np.arange(body * Gd), meta)
    if vb == 16:
        put16(VC, content["v_raw"])
    elif body:
        # stream (j, jp, n, vg) holds, at position VALUE_STREAM_POS[vb][e], the code of channel
        # 16 (2 vg + c div 2) + n, token 16 (c mod 2) + 8 jp + u of block j (e = 8 c + u)
        _, pos = value_maps(nblk, D, vb)
        j = np.arange(nblk)[:, None, None]
        c = np.arange(D)[None, :, None]
        i = np.arange(GROUP)[None, None, :]
        jp, n, vg = (i // 8) % 2, c % 16, (c // 16) // 2
        st = np.zeros((nblk, 2, 16, Gd, GROUP), dtype=np.uint8)
        st[j, jp, n, vg, pos] = np.asarray(content["v_codes"])
        words = pack_stream(st, vb)                                                 # [j][jp][n][vg][vb]
        jj = np.arange(nblk)[:, None, None, None]
        lane = 16 * (2 * (jj % 2) + np.arange(2)[None, :, None, None]) + np.arange(16)[None, None, :, None]
        first = ((jj // 2) * TILE + lane) * Gd * vb + np.arange(Gd)[None, None, None, :] * vb
        put32(VC, first[..., None] + np.arange(vb), words)
        meta = (content["v_s"].view(np.uint16).astype(np.uint32)
                | (content["v_z"].view(np.uint16).astype(np.uint32) << np.uint32(16)))
        put32(VM, value_meta_index(nblk, D), meta)
    if cfg.quant == "hybrid" and nblk:
        base = (np.arange(nblk) * 2 * Gd)[:, None]
        if kb != 16:
            kf = np.asarray(content["k_flag"]).reshape(nblk, GROUP * Gd)
            put32(FL, base + np.arange(Gd), _bits_to_words(kf))
        if vb != 16:
            put32(FL, base + Gd + np.arange(Gd), _bits_to_words(np.asarray(content["v_flag"])))
    put16(SK, content["sink_k"][:ns])
    put16(SV, content["sink_v"][:ns])
    R = ring_slots(cfg.n_recent)
    toks = np.arange(ns + body, T)
    slots = (toks - cfg.n_sink) % R
    for r, key in ((RK, "win_k"), (RV, "win_v")):
        buf = data[r].view(np.uint16).reshape(R, D)
        mk = mask[r].reshape(R, 2 * D)
        buf[slots] = content[key]
        mk[slots] = True
    if sz[KN]:
        data[KN][:] = np.asarray(content["k_norm"], dtype=np.float32).view(np.uint8)
        mask[KN][:] = True
    return data, mask


def oracle_head_content(oc, b: int, h: int) -> dict:
    """The logical content of (row b, KV head h) of an oracle cache, in decode_head's keys."""
    e = oc.heads[h]
    out = {}
    for key in ("k_codes", "k_s", "k_z", "k_flag", "v_codes", "v_s", "v_z", "v_flag", "k_raw", "v_raw"):
        if key in e:
            out[key] = e[key][b]
    out["sink_k"] = oc.sink_k[b, h]
    out["sink_v"] = oc.sink_v[b, h]
    out["win_k"] = oc.win_k[b, h]
    out["win_v"] = oc.win_v[b, h]
    if oc.k_norm is not None and oc.cfg.k_bits[h] != 16:
        out["k_norm"] = oc.k_norm[b, h]
    return out


def assert_content_equal(got: dict, want: dict, where=""):
    """Bit-exact comparison of two logical contents (float16 fields compared as bits)."""
    assert set(got) == set(want), (where, sorted(got), sorted(want))
    for key in want:
        a, b_ = np.asarray(got[key]), np.asarray(want[key])
        if a.dtype == np.float16:
            a, b_ = a.view(np.uint16), b_.view(np.uint16)
        elif a.dtype == np.float32:
            a, b_ = a.view(np.uint32), np.asarray(b_, dtype=np.float32).view(np.uint32)
        assert a.shape == b_.shape, (where, key, a.shape, b_.shape)
        bad = np.nonzero(a.reshape(-1) != b_.reshape(-1))[0]
        assert bad.size == 0, f"{where} {key}: {bad.size} of {a.size} differ (first at {bad[:4]})"
