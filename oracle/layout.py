"""Pool layout as a plain index function (test infrastructure only).

The pages fix only the logical structure: a pool of preallocated, fixed-size
physical blocks, each holding the K/V of ``block_size`` consecutive tokens, and
a per-sequence table mapping logical block i to a physical block
("KV Cache 原理与 PagedAttention", §三 工作方式 steps 1-2; aiworkagent.org Q17,
PagedAttention 的关键数据结构).  The byte layout inside the pool is this
library's own choice, documented in ``include/pkv.h``; this module restates that
documentation as arithmetic so that the oracle can read and write pools
produced by the device code.

Element offsets below are in *elements* of the storage type (bf16: 2 bytes,
fp8/int8: 1 byte) from the start of the K (or V) region:

    K:  ((((layer * NB + block) * Hkv + head) * B * D)
          + ((d // X) * B + t) * X + (d % X))          X = 16 // elem_bytes
    V:  ((((layer * NB + block) * Hkv + head) * B * D)
          + ((t // 4) * D + d) * 4 + (t % 4))
    K/V scales (INT8 per token-head, fp32 elements):
          ((layer * NB + block) * Hkv + head) * B + t
    K/V channel scales (INT8 per channel, fp32 elements, set by the caller):
          (layer * Hkv + head) * D + d
    INT8 with per-channel K and per-tensor V scales keeps the K channel
    scales only (same index); the call passes the V scale.
    INT8 per tensor and FP8 keep no scales in the pool (the call passes them).

INT4 (per-channel calibrated scales, as INT8 per channel) packs two codes per
byte and has its own index functions, in *nibbles* from the start of the
region (byte nibble // 2, low half when nibble is even).  With P = D / 8 bytes
per piece and, inside a 32-bit word, nibble n at bits 4n .. 4n + 3:

    K:  tile nibble 2 * ((j * B + t) * P + 4 * kk) + n
          kk = d // 32, j = (d % 32) // 8, i = d % 8, n = 4 * (i % 2) + i // 2
        (word kk of piece (j, t) holds dims 32 kk + 8 j .. + 7 of token t)
    V:  tile nibble 2 * ((g * 16 + m) * P + 4 * (c // 2)) + n
          g = t // 4, r = t % 4, c = d // 16, m = d % 16,
          n = 4 * (r % 2) + 2 * (r // 2) + c % 2
        (word c // 2 of piece (g, m) holds dims 16 c + m of tiles c = 2w, 2w+1
         for the 4 tokens of group g; each byte holds one token's two dims)

with tile nibble 0 at tile_base * 2.  A stored nibble is the code plus 8.

Regions are laid out K, V, K-scales, V-scales (those that exist), each
starting at a multiple of 256 bytes from the pool base.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

KV_BF16, KV_FP8_E5M2, KV_INT8, KV_INT8_TENSOR, KV_INT8_CHANNEL, KV_INT4 = 0, 1, 2, 3, 4, 5
# INT8 codes with K per channel (the pool's scales) and V per tensor (the
# call's scale): K and V quantised at different granularities
KV_INT8_KCHANNEL_VTENSOR = 6
# bytes of one entry of the storage array (INT4: one byte holds two codes)
ELEM_BYTES = {KV_BF16: 2, KV_FP8_E5M2: 1, KV_INT8: 1, KV_INT8_TENSOR: 1, KV_INT8_CHANNEL: 1, KV_INT4: 1,
              KV_INT8_KCHANNEL_VTENSOR: 1}
INT8_CODES = (KV_INT8, KV_INT8_TENSOR, KV_INT8_CHANNEL, KV_INT8_KCHANNEL_VTENSOR)
REGION_ALIGN = 256


@dataclass(frozen=True)
class PoolShape:
    num_layers: int
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: int = KV_BF16

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.kv_dtype]

    @property
    def x(self) -> int:
        return 16 // self.elem_bytes

    @property
    def tile_elems(self) -> int:
        return self.block_size * self.head_dim

    @property
    def tile_units(self) -> int:
        """Entries of the storage array per (block, head) tile."""
        return self.tile_elems // 2 if self.kv_dtype == KV_INT4 else self.tile_elems

    @property
    def region_elems(self) -> int:
        return self.num_layers * self.num_blocks * self.num_kv_heads * self.tile_elems

    @property
    def region_units(self) -> int:
        return self.num_layers * self.num_blocks * self.num_kv_heads * self.tile_units

    @property
    def has_scales(self) -> bool:
        """Per (token, head) scales stored beside each block's codes."""
        return self.kv_dtype == KV_INT8

    @property
    def has_channel_scales(self) -> bool:
        """Per (layer, head, dim) scales for K and for V, one region each."""
        return self.kv_dtype in (KV_INT8_CHANNEL, KV_INT4)

    @property
    def has_k_channel_scales(self) -> bool:
        """Per (layer, head, dim) K scales in the pool (V's may differ)."""
        return self.has_channel_scales or self.kv_dtype == KV_INT8_KCHANNEL_VTENSOR

    @property
    def has_v_scales(self) -> bool:
        """The pool holds a V scale region (beside the K one)."""
        return self.has_scales or self.has_channel_scales

    @property
    def scale_elems(self) -> int:
        """Elements of the K scale region (and of the V one, when it exists)."""
        if self.has_scales:
            return self.num_layers * self.num_blocks * self.num_kv_heads * self.block_size
        if self.has_k_channel_scales:
            return self.num_layers * self.num_kv_heads * self.head_dim
        return 0


def _align(n: int) -> int:
    return (n + REGION_ALIGN - 1) // REGION_ALIGN * REGION_ALIGN


def region_offsets(p: PoolShape):
    """Byte offsets (k, v, k_scale, v_scale, total).  Scale offsets are None
    when the storage type keeps no scales in the pool."""
    kv_bytes = p.region_units * p.elem_bytes
    k_off = 0
    v_off = _align(k_off + kv_bytes)
    end = _align(v_off + kv_bytes)
    if p.scale_elems:
        s_bytes = p.scale_elems * 4
        ks_off = end
        end = _align(ks_off + s_bytes)
        vs_off = None
        if p.has_v_scales:
            vs_off = end
            end = _align(vs_off + s_bytes)
        return k_off, v_off, ks_off, vs_off, end
    return k_off, v_off, None, None, end


def tile_base(p: PoolShape, layer, block, head):
    """First storage-array entry of the (layer, block, head) tile."""
    return (((np.asarray(layer, dtype=np.int64) * p.num_blocks + block)
             * p.num_kv_heads + head) * p.tile_units)


def int4_k_nibble(p: PoolShape, layer, block, head, t, d):
    """Nibble index (from the region start) of INT4 K element (t, d)."""
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    piece = p.head_dim // 8
    kk, j, i = d // 32, (d % 32) // 8, d % 8
    n = 4 * (i % 2) + i // 2
    return 2 * tile_base(p, layer, block, head) + 2 * ((j * p.block_size + t) * piece + 4 * kk) + n


def int4_v_nibble(p: PoolShape, layer, block, head, t, d):
    """Nibble index (from the region start) of INT4 V element (t, d)."""
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    piece = p.head_dim // 8
    g, r, c, m = t // 4, t % 4, d // 16, d % 16
    n = 4 * (r % 2) + 2 * (r // 2) + c % 2
    return 2 * tile_base(p, layer, block, head) + 2 * ((g * 16 + m) * piece + 4 * (c // 2)) + n


def read_nibbles(region: np.ndarray, nib) -> np.ndarray:
    """Stored nibbles (0..15) at the given nibble indices of a byte region."""
    nib = np.asarray(nib, dtype=np.int64)
    b = region[nib >> 1].astype(np.int64)
    return np.where(nib & 1, b >> 4, b & 15)


def write_nibbles(region: np.ndarray, nib, vals) -> None:
    """Store nibbles (0..15) at the given nibble indices (distinct) of a byte region."""
    nib = np.asarray(nib, dtype=np.int64).ravel()
    vals = np.asarray(vals, dtype=np.int64).ravel()
    hi = (nib & 1) == 1
    for sel, shift, keep in ((~hi, 0, 0xF0), (hi, 4, 0x0F)):
        idx = nib[sel] >> 1
        region[idx] = (region[idx] & keep) | ((vals[sel] & 15) << shift)


def k_offset(p: PoolShape, layer, block, head, t, d):
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    return tile_base(p, layer, block, head) + ((d // p.x) * p.block_size + t) * p.x + (d % p.x)


def v_offset(p: PoolShape, layer, block, head, t, d):
    t = np.asarray(t, dtype=np.int64)
    d = np.asarray(d, dtype=np.int64)
    return tile_base(p, layer, block, head) + ((t // 4) * p.head_dim + d) * 4 + (t % 4)


def scale_offset(p: PoolShape, layer, block, head, t):
    return ((np.asarray(layer, dtype=np.int64) * p.num_blocks + block)
            * p.num_kv_heads + head) * p.block_size + np.asarray(t, dtype=np.int64)


def channel_scale_offset(p: PoolShape, layer, head, d):
    return (np.asarray(layer, dtype=np.int64) * p.num_kv_heads + head) * p.head_dim + np.asarray(d, dtype=np.int64)


def k_tiles_as_tokens(p: PoolShape, region: np.ndarray, layer: int, blocks) -> np.ndarray:
    """K of the listed blocks of one layer as [len(blocks) * B, Hkv, D],
    token-major, in storage elements.  Each (block, head) tile is contiguous
    and, by the K formula above, is the array [D / X][B][X] (piece, token,
    lane); putting the token axis first and merging piece and lane gives
    [B][D]."""
    blocks = np.asarray(blocks, dtype=np.int64)
    if p.kv_dtype == KV_INT4:
        return _int4_k_tiles(p, region, layer, blocks)
    t = region.reshape(p.num_layers, p.num_blocks, p.num_kv_heads,
                       p.head_dim // p.x, p.block_size, p.x)[layer][blocks]
    # [nb, H, D/X, B, X] -> [nb, B, H, D/X, X]
    t = t.transpose(0, 3, 1, 2, 4)
    return t.reshape(blocks.size * p.block_size, p.num_kv_heads, p.head_dim)


def v_tiles_as_tokens(p: PoolShape, region: np.ndarray, layer: int, blocks) -> np.ndarray:
    """V of the listed blocks as [len(blocks) * B, Hkv, D]: by the V formula a
    tile is the array [B / 4][D][4] (token group, dim, token in group)."""
    blocks = np.asarray(blocks, dtype=np.int64)
    if p.kv_dtype == KV_INT4:
        return _int4_v_tiles(p, region, layer, blocks)
    t = region.reshape(p.num_layers, p.num_blocks, p.num_kv_heads,
                       p.block_size // 4, p.head_dim, 4)[layer][blocks]
    # [nb, H, B/4, D, 4] -> [nb, B/4, 4, H, D]
    t = t.transpose(0, 2, 4, 1, 3)
    return t.reshape(blocks.size * p.block_size, p.num_kv_heads, p.head_dim)


def _words_as_nibbles(words: np.ndarray) -> np.ndarray:
    """uint8 [..., 4] little-endian 32-bit words -> nibbles [..., 8], n-th
    nibble at bits 4n .. 4n + 3."""
    lo = words & 15
    hi = words >> 4
    # byte b holds nibbles 2b (low half) and 2b + 1 (high half)
    return np.stack([lo, hi], axis=-1).reshape(words.shape[:-1] + (8,))


def _int4_k_tiles(p: PoolShape, region: np.ndarray, layer: int, blocks: np.ndarray) -> np.ndarray:
    """Stored K nibbles as [len(blocks) * B, Hkv, D]: a tile is the byte array
    [4 (j)][B (t)][D / 32 (kk)][4], and word kk's nibble n is element
    i = 2 (n % 4) + n // 4 of dims 32 kk + 8 j .. + 7."""
    B, D, H = p.block_size, p.head_dim, p.num_kv_heads
    t = region.reshape(p.num_layers, p.num_blocks, H, 4, B, D // 32, 4)[layer][blocks]
    nib = _words_as_nibbles(t.astype(np.int64))                 # [nb, H, 4j, B, KK, 8n]
    i_of_n = np.array([2 * (n % 4) + n // 4 for n in range(8)])
    byi = np.empty_like(nib)
    byi[..., i_of_n] = nib                                       # element order i
    # [nb, H, j, B, kk, i] -> [nb, B, H, kk, j, i]: dim = 32 kk + 8 j + i
    out = byi.transpose(0, 3, 1, 4, 2, 5)
    return out.reshape(blocks.size * B, H, D)


def _int4_v_tiles(p: PoolShape, region: np.ndarray, layer: int, blocks: np.ndarray) -> np.ndarray:
    """Stored V nibbles as [len(blocks) * B, Hkv, D]: a tile is the byte array
    [B / 4 (g)][16 (m)][D / 32 (w)][4], and word w's nibble n is token
    r = n // 4 + 2 ((n // 2) % 2) of the group and tile c = 2 w + n % 2 (dim
    16 c + m)."""
    B, D, H = p.block_size, p.head_dim, p.num_kv_heads
    t = region.reshape(p.num_layers, p.num_blocks, H, B // 4, 16, D // 32, 4)[layer][blocks]
    nib = _words_as_nibbles(t.astype(np.int64))                 # [nb, H, g, m, w, 8n]
    out = np.empty((blocks.size, H, B // 4, 4, D // 16, 16), dtype=np.int64)   # [.., g, r, c, m]
    for n in range(8):
        r = n // 4 + 2 * ((n // 2) % 2)
        for w in range(D // 32):
            out[:, :, :, r, 2 * w + n % 2, :] = nib[:, :, :, :, w, n]
    # [nb, H, g, r, c, m] -> [nb, g, r, H, c, m]
    return out.transpose(0, 2, 3, 1, 4, 5).reshape(blocks.size * B, H, D)


def scales_as_tokens(p: PoolShape, region: np.ndarray, layer: int, blocks) -> np.ndarray:
    """Per-token-head scales of the listed blocks as [len(blocks) * B, Hkv]."""
    blocks = np.asarray(blocks, dtype=np.int64)
    t = region.reshape(p.num_layers, p.num_blocks, p.num_kv_heads, p.block_size)[layer][blocks]
    return t.transpose(0, 2, 1).reshape(blocks.size * p.block_size, p.num_kv_heads)


# ------------------------------------------------------------ host pool image
@dataclass
class PoolImage:
    """Host copy of a whole pool, split into typed flat regions."""
    shape: PoolShape
    k: np.ndarray                 # uint16 (bf16 bits) or uint8 / int8 codes
    v: np.ndarray
    k_scale: np.ndarray | None    # float32
    v_scale: np.ndarray | None

    def copy(self) -> "PoolImage":
        return PoolImage(self.shape, self.k.copy(), self.v.copy(),
                         None if self.k_scale is None else self.k_scale.copy(),
                         None if self.v_scale is None else self.v_scale.copy())


def _storage_dtype(p: PoolShape):
    return {KV_BF16: np.uint16, KV_FP8_E5M2: np.uint8, KV_INT8: np.int8, KV_INT8_TENSOR: np.int8,
            KV_INT8_CHANNEL: np.int8, KV_INT4: np.uint8, KV_INT8_KCHANNEL_VTENSOR: np.int8}[p.kv_dtype]


def empty_image(p: PoolShape, fill: int = 0) -> PoolImage:
    dt = _storage_dtype(p)
    k = np.full(p.region_units, fill, dtype=dt)
    v = np.full(p.region_units, fill, dtype=dt)
    ks = vs = None
    if p.scale_elems:
        ks = np.zeros(p.scale_elems, dtype=np.float32)
        if p.has_v_scales:
            vs = np.zeros(p.scale_elems, dtype=np.float32)
    return PoolImage(p, k, v, ks, vs)


def image_from_bytes(p: PoolShape, raw: np.ndarray) -> PoolImage:
    """Split the raw bytes of a whole pool (uint8) into its typed regions."""
    raw = np.asarray(raw, dtype=np.uint8)
    k_off, v_off, ks_off, vs_off, total = region_offsets(p)
    assert raw.size >= total, (raw.size, total)
    nb = p.region_units * p.elem_bytes
    dt = _storage_dtype(p)
    k = raw[k_off:k_off + nb].view(dt).copy()
    v = raw[v_off:v_off + nb].view(dt).copy()
    ks = vs = None
    if p.scale_elems:
        sb = p.scale_elems * 4
        ks = raw[ks_off:ks_off + sb].view(np.float32).copy()
        if vs_off is not None:
            vs = raw[vs_off:vs_off + sb].view(np.float32).copy()
    return PoolImage(p, k, v, ks, vs)


def image_to_bytes(img: PoolImage) -> np.ndarray:
    p = img.shape
    k_off, v_off, ks_off, vs_off, total = region_offsets(p)
    raw = np.zeros(total, dtype=np.uint8)
    kb = img.k.view(np.uint8)
    raw[k_off:k_off + kb.size] = kb
    vb = img.v.view(np.uint8)
    raw[v_off:v_off + vb.size] = vb
    if p.scale_elems:
        ksb = img.k_scale.view(np.uint8)
        raw[ks_off:ks_off + ksb.size] = ksb
        if vs_off is not None:
            vsb = img.v_scale.view(np.uint8)
            raw[vs_off:vs_off + vsb.size] = vsb
    return raw
