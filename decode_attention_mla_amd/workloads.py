"""Seeded synthetic inputs for dense and sparse MLA decode.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  Both the CPU oracle (tests) and the GPU path consume what it
returns, so the two sides always see bit-identical bf16 data.

Shapes follow the problem statement on the FlashMLA overview page
("[DeepSeek-3] FlashMLA", section 3, tensor shapes for dense decode):

    q             [batch, s_q, h_q, 576]            bf16
    kv_cache      [num_blocks, 64, 1, 576]           bf16 (K = all 576, V = first 512)
    block_table   [batch, max_blocks_per_seq]        int32
    cache_seqlens [batch]                            int32

bf16 tensors are carried as numpy ``uint16`` bit patterns.

Recipe (all seeded by ``numpy.random.default_rng(seed)``), in draw order:
  1. sequence lengths (fixed lists, or integers uniform on [lo, hi] inclusive);
  2. a random permutation of the physical page pool; pages are dealt to the
     requests in order, no page is shared between requests;
  3. q as fp32 N(0,1) rounded to bf16 (round to nearest even);
  4. the whole page pool as fp32 N(0,1) rounded to bf16.
Then every byte the method must never read is overwritten with a poison
value: unused pages, the tail tokens of each request's last page
(token >= L), and the padding entries of the block table, which point at an
unused (poisoned) page.  A leak through any of these shows as a gross error.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PAGE = 64          # tokens per KV page
D_QK = 576         # 512 latent + 64 RoPE dims, used by QK^T
D_V = 512          # latent dims, used by PV
POISON = 1.0e4     # fp32 value written where no read may land (bf16 -> 9984)
SOFTMAX_SCALE = float(np.float32(192.0 ** -0.5))  # original q head = 128 + 64 dims


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


POISON_BITS = int(f32_to_bf16_bits(np.array([POISON], np.float32))[0])


@dataclasses.dataclass
class MlaInputs:
    name: str
    q: np.ndarray             # uint16 [b, s_q, h_q, 576]
    kv_cache: np.ndarray      # uint16 [num_blocks, 64, 1, 576]
    block_table: np.ndarray   # int32 [b, max_blocks]
    cache_seqlens: np.ndarray  # int32 [b]
    softmax_scale: float

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


# The five synthetic workloads (tiny parity case, TP-sharded memory-bound
# decode, compute-bound decode, ragged MTP decode, long-context decode).
CONFIGS = {
    1: dict(name="tiny_b2_hq16_L100_257", batch=2, s_q=1, h_q=16, seqlens=[100, 257],
            pool=16, max_blocks=5),
    2: dict(name="membound_b16_hq16_L1024-4096", batch=16, s_q=1, h_q=16, seqlens=(1024, 4096),
            pool=1024, max_blocks=64),
    3: dict(name="compute_b64_hq128_L4096", batch=64, s_q=1, h_q=128, seqlens=[4096] * 64,
            pool=4096, max_blocks=64),
    4: dict(name="mtp_b128_sq2_hq128_L512-16384", batch=128, s_q=2, h_q=128,
            seqlens=(512, 16384), pool=None, max_blocks=256),
    5: dict(name="long_b2_hq128_L131072_65537", batch=2, s_q=1, h_q=128,
            seqlens=[131072, 65537], pool=3073, max_blocks=2048),
}


def _draw_normal_bf16(rng: np.random.Generator, shape, chunk_elems: int = 1 << 24) -> np.ndarray:
    """fp32 N(0,1) draws rounded to bf16, generated in fixed-size chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def make_inputs(batch: int, s_q: int, h_q: int, seqlens, pool: int | None, max_blocks: int,
                seed: int, softmax_scale: float = SOFTMAX_SCALE, name: str = "custom",
                tail_poison: float = POISON) -> MlaInputs:
    """Draw one seeded workload following the recipe in the module docstring.

    ``seqlens`` is a list of lengths or a ``(lo, hi)`` pair for integers
    uniform on [lo, hi].  ``pool`` is the physical page count; it is raised,
    if needed, so that at least one page stays unused (the poisoned target of
    block-table padding).
    """
    rng = np.random.default_rng(seed)
    if isinstance(seqlens, tuple):
        lo, hi = seqlens
        lens = rng.integers(lo, hi + 1, size=batch).astype(np.int32)
    else:
        lens = np.asarray(seqlens, dtype=np.int32)
        assert lens.shape == (batch,)
    npages = [(int(L) + PAGE - 1) // PAGE for L in lens]
    need = sum(npages)
    if max(npages, default=0) > max_blocks:
        raise ValueError("a sequence needs more pages than max_blocks")
    pool = max(pool or 0, need + 1)
    perm = rng.permutation(pool).astype(np.int32)
    spare = int(perm[need])  # first unused page: target of block-table padding
    block_table = np.full((batch, max_blocks), spare, dtype=np.int32)
    at = 0
    for b, n in enumerate(npages):
        block_table[b, :n] = perm[at:at + n]
        at += n
    q = _draw_normal_bf16(rng, (batch, s_q, h_q, D_QK))
    kv = _draw_normal_bf16(rng, (pool, PAGE, 1, D_QK))
    poison = int(f32_to_bf16_bits(np.array([tail_poison], np.float32))[0])
    used = np.zeros(pool, dtype=bool)
    used[perm[:need]] = True
    kv[~used] = poison
    for b, n in enumerate(npages):
        tail = int(lens[b]) - (n - 1) * PAGE
        if n and tail < PAGE:
            kv[block_table[b, n - 1], tail:] = poison
    return MlaInputs(name=name, q=q, kv_cache=kv, block_table=block_table,
                     cache_seqlens=lens, softmax_scale=float(softmax_scale))


@dataclasses.dataclass
class SparseInputs:
    """Sparse (top-k) decode inputs ("[DeepSeek-3] FlashMLA", section 11)."""
    name: str
    q: np.ndarray             # uint16 [b, s_q, h_q, 576]
    kv_cache: np.ndarray      # uint16 [num_blocks, 64, 1, 576]
    indices: np.ndarray       # int32 [b, s_q, topk]: page_id * 64 + offset, -1 = no key
    topk_length: np.ndarray | None   # int32 [b] or None (all topk entries count)
    softmax_scale: float

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def s_q(self) -> int:
        return int(self.q.shape[1])

    @property
    def h_q(self) -> int:
        return int(self.q.shape[2])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_cache.shape[0])


def make_sparse_inputs(batch: int, s_q: int, h_q: int, topk: int, context, seed: int,
                       pad_frac: float = 0.0, topk_length=None, softmax_scale: float = SOFTMAX_SCALE,
                       name: str = "sparse") -> SparseInputs:
    """Draw one seeded sparse workload.

    Recipe, in draw order: each request's context length (``context`` is a
    list or a ``(lo, hi)`` pair, uniform inclusive; at least ``topk``);
    a permutation of a page pool holding every context plus one spare page;
    q and the pool as fp32 N(0,1) rounded to bf16; then, per (request, query
    token), ``topk`` distinct positions of that request's context drawn
    uniformly without replacement (the output of a top-k selector over the
    context, in arbitrary order), mapped to page_id * 64 + offset through the
    request's pages.  With ``pad_frac`` > 0 that fraction of entries, at
    random places, becomes -1 (padding).  ``topk_length`` (a list, or
    None) is passed through.  Pool rows no list names are poisoned, so a
    wrong gather shows as a gross error.
    """
    rng = np.random.default_rng(seed)
    if isinstance(context, tuple):
        lo, hi = context
        ctx = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    else:
        ctx = np.asarray(context, dtype=np.int64)
        assert ctx.shape == (batch,)
    assert np.all(ctx >= topk)
    npages = [(int(L) + PAGE - 1) // PAGE for L in ctx]
    pool = sum(npages) + 1
    perm = rng.permutation(pool).astype(np.int64)
    q = _draw_normal_bf16(rng, (batch, s_q, h_q, D_QK))
    kv = _draw_normal_bf16(rng, (pool, PAGE, 1, D_QK))
    indices = np.empty((batch, s_q, topk), dtype=np.int32)
    at = 0
    for b in range(batch):
        pages = perm[at:at + npages[b]]
        at += npages[b]
        for s in range(s_q):
            pos = rng.choice(int(ctx[b]), size=topk, replace=False)
            indices[b, s] = (pages[pos // PAGE] * PAGE + pos % PAGE).astype(np.int32)
    if pad_frac > 0:
        indices[rng.random(indices.shape) < pad_frac] = -1
    named = np.zeros(pool * PAGE, dtype=bool)
    named[indices[indices >= 0].astype(np.int64)] = True
    flat = kv.reshape(pool * PAGE, D_QK)
    flat[~named] = int(f32_to_bf16_bits(np.array([POISON], np.float32))[0])
    tl = None if topk_length is None else np.asarray(topk_length, dtype=np.int32)
    return SparseInputs(name=name, q=q, kv_cache=kv, indices=indices, topk_length=tl,
                        softmax_scale=float(softmax_scale))


# The sparse workload of the pages' FP8-sparse micro-benchmark shape
# (batch 128, s_q 2, h_q 128, topk 2048; section 13 of the overview), here
# on a bf16 cache, each request's context 4096..8192 tokens.
SPARSE_CONFIG = dict(name="sparse_b128_sq2_hq128_topk2048", batch=128, s_q=2, h_q=128, topk=2048,
                     context=(4096, 8192))


def sparse_config_inputs(seed: int = 6) -> SparseInputs:
    c = SPARSE_CONFIG
    return make_sparse_inputs(c["batch"], c["s_q"], c["h_q"], c["topk"], c["context"], seed=seed, name=c["name"])


def sparse_algorithmic_work(indices: np.ndarray, h_q: int, topk_length=None,
                            kv_row_bytes: int = 2 * D_QK) -> tuple[float, float]:
    """(FLOPs, bytes) of one sparse decode call: every counted entry of every
    query token's list is one key (576 + 512 dims, 2 FLOPs each, h_q heads)
    and one cache row read (1152 bytes in bf16, 656 as an FP8 record);
    plus the index list (4 B per entry),
    q read, out written (bf16) and lse written (fp32)."""
    b, s_q, topk = indices.shape
    keys = 0
    for i in range(b):
        n = topk if topk_length is None else min(max(int(topk_length[i]), 0), topk)
        keys += int((indices[i, :, :n] >= 0).sum())
    rows = b * s_q * h_q
    flops = 2.0 * h_q * keys * (D_QK + D_V)
    nbytes = float(kv_row_bytes) * keys + 4.0 * b * s_q * topk + 2.0 * rows * (D_QK + D_V) + 4.0 * rows
    return flops, nbytes


# ---------------------------------------------------------------------------
# FP8 cache records ("[DeepSeek-3] FlashMLA", section 12): 656 bytes per token,
#   bytes   0 .. 511  the 512 latent dims as float8 e4m3 (OCP e4m3fn);
#   bytes 512 .. 527  four fp32 scales, scale i covering dims 128 i .. 128 i + 127;
#   bytes 528 .. 655  the 64 RoPE dims, bf16, not quantized.
FP8_RECORD = 656
FP8_MAX = 448.0


def quantize_e4m3(x: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """Round fp32 values to the nearest e4m3fn byte (ties to the even
    mantissa), saturating at +-448, by integer arithmetic on the fp32 bits
    (in chunks, so that the temporaries stay small).  Input generation only:
    the cache's writer quantizes, the method reads the bytes."""
    x = np.asarray(x, np.float32)
    if x.size > chunk:
        out = np.empty(x.shape, np.uint8)
        xf, of = x.reshape(-1), out.reshape(-1)
        for s in range(0, xf.size, chunk):
            of[s:s + chunk] = quantize_e4m3(xf[s:s + chunk], chunk)
        return out
    v = np.clip(x, -FP8_MAX, FP8_MAX)
    a = np.abs(v)
    bits = a.view(np.uint32)
    e0 = (bits >> 23).astype(np.int32) - 127          # unbiased fp32 exponent
    man = bits & 0x7FFFFF
    m3 = (man >> 20).astype(np.int32)                 # top 3 mantissa bits
    rem = man & 0xFFFFF
    m3 = m3 + ((rem > 0x80000) | ((rem == 0x80000) & ((m3 & 1) == 1)))   # round half to even
    e = e0 + (m3 >> 3)                                # mantissa carry into the exponent
    normal = ((e + 7) << 3) | (m3 & 7)
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)   # below 2^-6: multiples of 2^-9 (8 -> 2^-6)
    byte = np.where(e0 >= -6, normal, sub)
    sign = np.where(np.signbit(v) & (byte != 0), 0x80, 0)
    return (byte | sign).astype(np.uint8)


def to_fp8_records(kv_bf16: np.ndarray, pages_per_chunk: int = 256) -> np.ndarray:
    """FP8 records of a bf16 cache [nb, 64, 1, 576]: per token and 128-dim
    tile, scale = fp32(max |x| / 448) (1 for an all-zero tile), bytes =
    e4m3(fp32(x / scale)); RoPE dims copied.  Returns uint8 [nb, 64, 1, 656]."""
    nb = kv_bf16.shape[0]
    rec = np.empty((nb, PAGE, FP8_RECORD), np.uint8)
    for p0 in range(0, nb, pages_per_chunk):
        p1 = min(nb, p0 + pages_per_chunk)
        bits = kv_bf16[p0:p1].reshape(p1 - p0, PAGE, D_QK)
        lat = bf16_bits_to_f32(bits[..., :D_V]).reshape(p1 - p0, PAGE, 4, 128)
        amax = np.abs(lat).max(axis=-1)
        scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        rec[p0:p1, :, :D_V] = quantize_e4m3(lat / scale[..., None]).reshape(p1 - p0, PAGE, D_V)   # fp32 division
        rec[p0:p1, :, D_V:D_V + 16] = scale.view(np.uint8).reshape(p1 - p0, PAGE, 16)
        rec[p0:p1, :, D_V + 16:] = np.ascontiguousarray(bits[..., D_V:]).view(np.uint8).reshape(p1 - p0, PAGE, 128)
    return rec.reshape(nb, PAGE, 1, FP8_RECORD)


def config_inputs(index: int) -> MlaInputs:
    """Workload ``index`` (1..5) with seed ``index``."""
    c = CONFIGS[index]
    return make_inputs(c["batch"], c["s_q"], c["h_q"], c["seqlens"], c["pool"],
                       c["max_blocks"], seed=index, name=c["name"])


def algorithmic_work(seqlens, s_q: int, h_q: int, causal: bool = False, kv_row_bytes: int = 2 * D_QK) -> tuple[float, float]:
    """(FLOPs, bytes) the method must do for one decode call.

    FLOPs = 2 * h_q * sum over (request, query token) of the keys it sees *
    (576 + 512): the QK^T and PV products (all L keys, or with the causal
    mask L - (s_q - 1 - s) for query token s).  Bytes = bf16 KV read once per
    request (1152 bytes a token in bf16, 656 as an FP8 record), q read,
    out written (bf16), lse written (fp32).  Masked tail
    tokens, split partials and the block table are overhead and are not
    counted.
    """
    sl = np.asarray(seqlens, dtype=np.int64)
    R = s_q * h_q
    total = int(sl.sum())
    b = int(sl.shape[0])
    seen = s_q * total if not causal else int(sum(np.maximum(sl - (s_q - 1 - s), 0).sum() for s in range(s_q)))
    flops = 2.0 * h_q * seen * (D_QK + D_V)
    nbytes = float(kv_row_bytes) * total + 2.0 * (b * R * D_QK + b * R * D_V) + 4.0 * b * R
    return flops, nbytes


def pages_needed(L: int) -> int:
    return int(math.ceil(int(L) / PAGE))
