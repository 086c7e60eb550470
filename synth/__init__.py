"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only *makes bytes*: normal draws, rounding to binary16, and
packing draws into the 32-value q8_0 / q4_0 block formats that the cache is
stored in.  It holds none of the attention arithmetic and no dequantiser; the
oracle and the HIP library each read the bytes with their own code.

Cache layout (both sides read it through explicit byte strides): one tensor
per K and per V, position-major ``[n_keys][n_kv_heads][row]`` where a row is
the ``head_dim`` values of one (position, KV head) in the storage type.

Block formats ("F5 M6 -- PolyKV", S0 and the tier-family table): a block is
32 consecutive values along head_dim; q8_0 = binary16 scale + 32 signed bytes
(34 B); q4_0 = binary16 scale + 16 bytes of 4-bit codes (18 B), element i < 16
in the low nibble of byte i and element i >= 16 in the high nibble of byte
i - 16.  The quantiser rule used to *generate* blocks from normal draws is not
given by the pages; the one here (amax/127 for q8_0, signed-max/-8 for q4_0,
scale stored round-to-nearest-even) only shapes the test data.

TBQ3 (the 3-bit value tier) blocks are 128 values in 52 bytes: a binary16
norm, two zero bytes, 32 bytes of 2-bit magnitude indices, 16 bytes of sign
bits.  They are drawn here directly, without the tier's rotation or codebook:
the norm is that of 128 N(0,1) draws (rounded to binary16) and the indices
and sign bits are uniform random bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

F32, F16, Q8_0, Q4_0, TBQ3 = 0, 1, 2, 3, 4
TYPE_NAMES = {F32: "f32", F16: "f16", Q8_0: "q8_0", Q4_0: "q4_0", TBQ3: "tbq3"}
TYPE_BY_NAME = {v: k for k, v in TYPE_NAMES.items()}


def row_bytes(dtype: int, head_dim: int) -> int:
    """Bytes of one (position, KV head) row of ``head_dim`` values."""
    if dtype == F32:
        return 4 * head_dim
    if dtype == F16:
        return 2 * head_dim
    if dtype == TBQ3:
        if head_dim % 128:
            raise ValueError("tbq3 needs head_dim % 128 == 0")
        return head_dim // 128 * 52
    if head_dim % 32:
        raise ValueError("block types need head_dim % 32 == 0")
    if dtype == Q8_0:
        return head_dim // 32 * 34
    if dtype == Q4_0:
        return head_dim // 32 * 18
    raise ValueError(f"unknown dtype {dtype}")


def stream_seed(base: int, tensor_id: int, layer: int = 0) -> int:
    """Independent seed per (configuration, tensor, layer)."""
    x = (base * 0x9E3779B1 + tensor_id * 0x85EBCA77 + layer * 0xC2B2AE3D + 0x27D4EB2F) & 0x7FFFFFFFFFFFFFFF
    x ^= x >> 29
    x = (x * 0xBF58476D1CE4E5B9) & 0x7FFFFFFFFFFFFFFF
    x ^= x >> 32
    return x


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, device="cpu") -> torch.Tensor:
    """i.i.d. N(0,1) float32 draws."""
    return torch.randn(*shape, generator=generator(seed, device), device=device, dtype=torch.float32)


def _round_half_away(x: torch.Tensor) -> torch.Tensor:
    return torch.sign(x) * torch.floor(x.abs() + 0.5)


def pack_q8_0(x: torch.Tensor) -> torch.Tensor:
    """Pack float32 draws [..., D] into q8_0 blocks -> uint8 [..., D/32*34]."""
    *lead, d = x.shape
    xb = x.reshape(-1, 32).to(torch.float32)
    amax = xb.abs().amax(dim=1)
    scale = amax / 127.0
    inv = torch.where(scale > 0, 1.0 / torch.where(scale > 0, scale, torch.ones_like(scale)), torch.zeros_like(scale))
    q = _round_half_away(xb * inv[:, None]).clamp_(-127, 127).to(torch.int8)
    out = torch.empty(xb.shape[0], 34, dtype=torch.uint8, device=x.device)
    out[:, 0:2] = scale.to(torch.float16).view(torch.uint8).reshape(-1, 2)
    out[:, 2:] = q.view(torch.uint8)
    return out.reshape(*lead, d // 32 * 34)


def pack_q4_0(x: torch.Tensor) -> torch.Tensor:
    """Pack float32 draws [..., D] into q4_0 blocks -> uint8 [..., D/32*18]."""
    *lead, d = x.shape
    xb = x.reshape(-1, 32).to(torch.float32)
    idx = xb.abs().argmax(dim=1, keepdim=True)
    m = torch.gather(xb, 1, idx).squeeze(1)
    scale = m / -8.0
    inv = torch.where(scale != 0, 1.0 / torch.where(scale != 0, scale, torch.ones_like(scale)), torch.zeros_like(scale))
    n = torch.clamp(torch.trunc(xb * inv[:, None] + 8.5), 0, 15).to(torch.uint8)
    out = torch.empty(xb.shape[0], 18, dtype=torch.uint8, device=x.device)
    out[:, 0:2] = scale.to(torch.float16).view(torch.uint8).reshape(-1, 2)
    out[:, 2:] = n[:, :16] | (n[:, 16:] << 4)
    return out.reshape(*lead, d // 32 * 18)


def encode(x: torch.Tensor, dtype: int) -> torch.Tensor:
    """Store float32 draws [..., D] in ``dtype``; returns the storage tensor
    ([..., D] float32 / float16, or [..., row_bytes] uint8 for block types)."""
    if dtype == F32:
        return x.to(torch.float32).contiguous()
    if dtype == F16:
        return x.to(torch.float16).contiguous()
    if dtype == Q8_0:
        return pack_q8_0(x)
    if dtype == Q4_0:
        return pack_q4_0(x)
    raise ValueError(f"no packer for dtype {dtype}")


def draw_tbq3(n_keys: int, n_kv_heads: int, head_dim: int, g: torch.Generator, device) -> torch.Tensor:
    """TBQ3 rows drawn directly: uint8 [n_keys][n_kv_heads][head_dim/128*52]."""
    nb = head_dim // 128
    x = torch.randn(n_keys, n_kv_heads, nb, 128, generator=g, device=device, dtype=torch.float32)
    norm = x.double().norm(dim=-1).to(torch.float16)
    del x
    out = torch.zeros(n_keys, n_kv_heads, nb, 52, dtype=torch.uint8, device=device)
    out[..., 0:2] = norm.view(torch.uint8).reshape(n_keys, n_kv_heads, nb, 2)
    out[..., 4:52] = torch.randint(0, 256, (n_keys, n_kv_heads, nb, 48), generator=g, device=device, dtype=torch.uint8)
    return out.reshape(n_keys, n_kv_heads, nb * 52)


@dataclass
class Cache:
    """One K or V tensor, position-major [n_keys][n_kv_heads][row]."""

    data: torch.Tensor
    dtype: int
    n_keys: int
    n_kv_heads: int
    head_dim: int

    @property
    def row_bytes(self) -> int:
        return row_bytes(self.dtype, self.head_dim)

    @property
    def head_stride(self) -> int:
        return self.row_bytes

    @property
    def pos_stride(self) -> int:
        return self.n_kv_heads * self.row_bytes

    def to(self, device) -> "Cache":
        return Cache(self.data.to(device), self.dtype, self.n_keys, self.n_kv_heads, self.head_dim)

    def ptr(self, pos: int = 0) -> int:
        return self.data.data_ptr() + pos * self.pos_stride


def make_cache(n_keys: int, n_kv_heads: int, head_dim: int, dtype: int, seed: int, device="cpu",
               outlier_channels: int = 0, outlier_gain: float = 8.0, chunk_keys: int = 1 << 16,
               channels_seed: int | None = None, pinned: bool = False) -> Cache:
    """A cache tensor of N(0,1) draws stored in ``dtype``.

    ``outlier_channels`` (kv_head, d) channels, chosen without replacement from
    ``channels_seed`` (default ``seed``), are multiplied by ``outlier_gain``
    after rounding to the storage type (exact for a power of two gain on
    binary16 data).  Draws are made in key chunks to bound peak memory; the
    chunk size is part of the recipe (the same seed and chunk give the same
    bytes on the same device type).  ``pinned`` places the result in pinned
    host memory (device must be "cpu").
    """
    rb = row_bytes(dtype, head_dim)
    shape_tail = (n_kv_heads, head_dim) if dtype in (F32, F16) else (n_kv_heads, rb)
    tdtype = {F32: torch.float32, F16: torch.float16}.get(dtype, torch.uint8)
    out = torch.empty((n_keys,) + shape_tail, dtype=tdtype, device=device, pin_memory=pinned)
    g = generator(seed, device)
    for c0 in range(0, n_keys, chunk_keys):
        c1 = min(n_keys, c0 + chunk_keys)
        if dtype == TBQ3:
            out[c0:c1] = draw_tbq3(c1 - c0, n_kv_heads, head_dim, g, device)
            continue
        x = torch.randn(c1 - c0, n_kv_heads, head_dim, generator=g, device=device, dtype=torch.float32)
        out[c0:c1] = encode(x, dtype)
        del x
    if outlier_channels:
        if dtype not in (F32, F16):
            raise ValueError("outlier channels are defined for float storage only")
        gc = generator(seed if channels_seed is None else channels_seed, "cpu")
        sel = torch.randperm(n_kv_heads * head_dim, generator=gc)[:outlier_channels]
        hh, dd = (sel // head_dim).tolist(), (sel % head_dim).tolist()
        for h, d in zip(hh, dd):
            out[:, h, d] *= outlier_gain
    return Cache(out, dtype, n_keys, n_kv_heads, head_dim)


def make_query(n_seq: int, n_q_heads: int, head_dim: int, seed: int, device="cpu") -> torch.Tensor:
    """Query [n_seq][n_q_heads][head_dim] float32 N(0,1)."""
    return normal((n_seq, n_q_heads, head_dim), seed, device)


def append_rows(n_tokens: int, n_kv_heads: int, head_dim: int, seed: int, device="cpu",
                large: bool = True) -> torch.Tensor:
    """New K or V rows to append: binary32 [n_tokens][n_kv_heads][head_dim].

    N(0,1) draws, with planted 32-value blocks that exercise the storage
    rules: zero blocks, blocks scaled by 2^-20 (block scales in binary16's
    subnormal range) or 2^10, blocks on a quarter grid (many values exactly
    half-way between codes), and blocks whose largest magnitude occurs twice
    (same and opposite sign).  Which blocks are planted is drawn from the
    seed; the values are exact binary32 numbers.  large=False leaves the
    2^10-scaled blocks at N(0,1) scale (rows for attention checks: an absolute
    tolerance on O presumes values of order one).
    """
    g = generator(seed, "cpu")
    x = torch.randn(n_tokens, n_kv_heads, head_dim, generator=g, dtype=torch.float32)
    blocks = x.view(-1, 32)
    kind = torch.randint(0, 8, (blocks.shape[0],), generator=g)
    blocks[kind == 1] = 0.0
    blocks[kind == 2] *= 2.0 ** -20
    if large:
        blocks[kind == 3] *= 2.0 ** 10
    blocks[kind == 4] = torch.round(blocks[kind == 4] * 4) / 4
    for b in torch.nonzero(kind >= 6).flatten().tolist():
        i, j = torch.randperm(32, generator=g)[:2].tolist()
        top = blocks[b].abs().max()
        blocks[b, i] = top
        blocks[b, j] = top if kind[b] == 6 else -top
    return x.to(device)


# Per-block magnitude factors of make_cache_wide (powers of two, so binary16
# rounding of float data is unaffected apart from range).  "small" factors put
# q8_0 / q4_0 block scales (amax/127, m/-8 of N(0,1) draws) in binary16's
# subnormal range; "big" ones push q8_0 scales past 512 and q4_0 scales past
# 8192, where d * code leaves binary16's range, while staying finite.
WIDE_FACTORS = {
    F32: ([2.0 ** -30, 2.0 ** -12, 1.0, 1.0], [2.0 ** 20, 2.0 ** 40]),
    F16: ([2.0 ** -20, 2.0 ** -12, 1.0, 1.0], [2.0 ** 10, 2.0 ** 13]),
    Q8_0: ([2.0 ** -18, 2.0 ** -12, 1.0, 1.0], [2.0 ** 14, 2.0 ** 16]),
    Q4_0: ([2.0 ** -15, 2.0 ** -10, 1.0, 1.0], [2.0 ** 15, 2.0 ** 16]),
}


def make_cache_wide(n_keys: int, n_kv_heads: int, head_dim: int, dtype: int, seed: int, device="cpu",
                    big_every: int = 3, neg128_frac: float = 1.0 / 16) -> Cache:
    """A cache of N(0,1) draws whose 32-value blocks are scaled by powers of two
    that span the storage type's range (WIDE_FACTORS): small factors anywhere,
    big ones only in the keys of every ``big_every``-th run of 64 keys (so some
    runs of keys hold only ordinary blocks).  For q8_0 a fraction
    ``neg128_frac`` of the code bytes is then set to -128, a legal code the
    quantiser never makes.  Generated on the CPU (bytes are then moved to
    ``device``); the recipe is part of the data."""
    g = generator(seed, "cpu")
    x = torch.randn(n_keys, n_kv_heads, head_dim, generator=g, dtype=torch.float32)
    small, big = WIDE_FACTORS[dtype]
    nb = head_dim // 32
    kind = torch.randint(0, len(small) + len(big), (n_keys, n_kv_heads, nb), generator=g)
    keys = torch.arange(n_keys)
    big_ok = ((keys // 64) % big_every == 0)[:, None, None]
    table = torch.tensor(small + big, dtype=torch.float32)
    kind = torch.where(big_ok | (kind < len(small)), kind, kind % len(small))
    f = table[kind]  # [n][H][nb]
    x = (x.view(n_keys, n_kv_heads, nb, 32) * f[..., None]).view(n_keys, n_kv_heads, head_dim)
    data = encode(x, dtype)
    if dtype == Q8_0 and neg128_frac > 0:
        codes = data.view(n_keys, n_kv_heads, nb, 34)[..., 2:]
        hit = torch.rand(codes.shape, generator=g) < neg128_frac
        codes[hit] = 0x80
    return Cache(data.to(device).contiguous(), dtype, n_keys, n_kv_heads, head_dim)


def make_query_scaled(n_seq: int, n_q_heads: int, head_dim: int, seed: int, row_log2: list, device="cpu") -> torch.Tensor:
    """make_query with row h of every sequence multiplied by 2^row_log2[h % len(row_log2)]."""
    q = normal((n_seq, n_q_heads, head_dim), seed, "cpu")
    f = torch.tensor([2.0 ** row_log2[h % len(row_log2)] for h in range(n_q_heads)], dtype=torch.float32)
    return (q * f[None, :, None]).to(device)

