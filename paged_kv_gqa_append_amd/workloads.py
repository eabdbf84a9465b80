"""Seeded synthetic inputs for paged GQA decode, KV append and chunked prefill.

This module only draws random numbers and lays out page tables.  It holds
none of the attention or rotary arithmetic, so both the HIP path and the
fp64 CPU checker can be fed from it without sharing any of the method.

Geometry follows the Llama-3.2-1B numbers on the tiny-vllm chapter
"Weight Loading and GPU Buffer Design" (section "Preallocating the 16 compute
buffers": NUM_Q_HEADS = 32, KV_DIM = 512, EMBEDDING_LENGTH = 2048, i.e. head
dim 64 and 8 KV heads) and the samir-vllm article (section "Gestion de la KV
cache et strategies de batching": a shared pool of 16-token pages, one block
table per sequence and per layer; section "Limitations": 2048-token context,
16 layers).

Storage layout (the pages do not fix one; see the header include/pa.h):
  k_pool, v_pool : [num_pages][8 kv heads][16 slots][64] bf16   (head-major page)
  q              : [num_seqs][32][64] bf16
  k_new, v_new   : [num_seqs][8][64] bf16
  block_tables   : [num_seqs][max_blocks] int32, -1 past the used pages
  context_lens   : [num_seqs] int32, counts the appended token (pos = L - 1)

bf16 tensors are kept as uint16 bit patterns in numpy; conversion from the
drawn float32 values is round-to-nearest-even (torch CPU ``.to(bfloat16)``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 64
PAGE_SIZE = 16
GROUP = NUM_Q_HEADS // NUM_KV_HEADS
ROPE_THETA = 500000.0
MAX_CONTEXT = 2048
KV_BYTES_PER_TOKEN_LAYER = 2 * NUM_KV_HEADS * HEAD_DIM * 2  # K + V, bf16 -> 2048
PAGE_ELEMS = NUM_KV_HEADS * PAGE_SIZE * HEAD_DIM              # 8192 bf16 = 16 KiB

# Tensor ids for the per-(config, layer, tensor) seed streams.
_T_Q, _T_KNEW, _T_VNEW, _T_KPOOL, _T_VPOOL, _T_LAYOUT, _T_LENS, _T_OUTLIER = range(8)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch CPU)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


@dataclass
class PagedCase:
    """One synthetic paged-attention workload (host copy, bf16 as uint16)."""

    name: str
    num_layers: int
    num_seqs: int
    max_blocks: int
    num_pages: int
    context_lens: np.ndarray            # int32 [B]
    block_tables: np.ndarray            # int32 [layers][B][max_blocks]
    q: np.ndarray                       # uint16 [layers][B][32][64] (pre-RoPE)
    k_new: np.ndarray                   # uint16 [layers][B][8][64] (pre-RoPE)
    v_new: np.ndarray                   # uint16 [layers][B][8][64]
    k_pool: Optional[np.ndarray]        # uint16 [P][8][16][64]
    v_pool: Optional[np.ndarray]
    scale: float = 1.0 / 8.0
    theta: float = ROPE_THETA
    seed: int = 0
    notes: str = ""
    # Per-page slot multipliers used by the device-side pool fill (None: all 1).
    outlier_slots: Optional[np.ndarray] = None  # int64 [n] flat (page*16+slot)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one full step reads: tokens attended x 2048 B x layers."""
        return int(self.context_lens.astype(np.int64).sum()) * KV_BYTES_PER_TOKEN_LAYER * self.num_layers


@dataclass
class PrefillCase:
    name: str
    num_seqs: int
    chunk_len: int
    max_blocks: int
    num_pages: int
    prefix_lens: np.ndarray             # int32 [B]
    block_tables: np.ndarray            # int32 [B][max_blocks]
    q: np.ndarray                       # uint16 [B][C][32][64] (pre-RoPE)
    k_chunk: np.ndarray                 # uint16 [B][C][8][64] (pre-RoPE)
    v_chunk: np.ndarray                 # uint16 [B][C][8][64]
    k_pool: np.ndarray                  # uint16 [P][8][16][64]
    v_pool: np.ndarray
    scale: float = 1.0 / 8.0
    theta: float = ROPE_THETA
    seed: int = 0


# ---------------------------------------------------------------------------
# page-table layouts
# ---------------------------------------------------------------------------

def pages_needed(lens: np.ndarray) -> np.ndarray:
    return (np.asarray(lens, dtype=np.int64) + PAGE_SIZE - 1) // PAGE_SIZE


def random_block_tables(rng: np.random.Generator, lens: np.ndarray, num_layers: int,
                        max_blocks: int, num_pages: int) -> np.ndarray:
    """Each (layer, seq, block) draws a distinct page id from the whole pool."""
    need = pages_needed(lens)
    total = int(need.sum()) * num_layers
    if total > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {total}")
    ids = rng.permutation(num_pages)[:total].astype(np.int32)
    bt = np.full((num_layers, len(lens), max_blocks), -1, dtype=np.int32)
    k = 0
    for layer in range(num_layers):
        for s, n in enumerate(need):
            bt[layer, s, :n] = ids[k:k + n]
            k += n
    return bt


def fragmented_block_tables(rng: np.random.Generator, lens: np.ndarray, num_layers: int,
                            max_blocks: int, num_pages: int, history: int = 4000) -> np.ndarray:
    """Page ids handed out by a LIFO free list after a random alloc/free history.

    Dummy requests of random size are admitted and retired in random order, so
    the free list ends up non-contiguous and non-monotonic, as in a serving
    engine that has run for a while.  The real sequences then allocate their
    pages, layer by layer, from that list.
    """
    free: List[int] = list(range(num_pages - 1, -1, -1))  # pop() yields 0, 1, 2, ...
    live: List[List[int]] = []
    for _ in range(history):
        if live and (rng.random() < 0.45 or len(free) < 256):
            victim = live.pop(int(rng.integers(len(live))))
            rng.shuffle(victim)
            free.extend(victim)
        else:
            n = int(rng.integers(1, 129))
            if n > len(free):
                continue
            live.append([free.pop() for _ in range(n)])
    for pages in live:  # retire whatever is still live, in random order
        rng.shuffle(pages)
        free.extend(pages)
    need = pages_needed(lens)
    if int(need.sum()) * num_layers > len(free):
        raise ValueError("pool too small for the ragged batch")
    bt = np.full((num_layers, len(lens), max_blocks), -1, dtype=np.int32)
    for layer in range(num_layers):
        for s, n in enumerate(need):
            bt[layer, s, :n] = [free.pop() for _ in range(int(n))]
    return bt


def used_slots(block_tables_layer: np.ndarray, lens: np.ndarray):
    """(page, slot) pairs that hold tokens 0..L-1 of each sequence of one layer."""
    out = []
    for s, L in enumerate(lens):
        t = np.arange(int(L))
        out.append((block_tables_layer[s, t // PAGE_SIZE].astype(np.int64), t % PAGE_SIZE))
    pages = np.concatenate([p for p, _ in out]) if out else np.zeros(0, np.int64)
    slots = np.concatenate([t for _, t in out]) if out else np.zeros(0, np.int64)
    return pages, slots


def poison_unused(pool: np.ndarray, block_tables: np.ndarray, lens: np.ndarray) -> None:
    """Write bf16 NaN into every slot no sequence uses (all layers)."""
    used = np.zeros((pool.shape[0], PAGE_SIZE), dtype=bool)
    for layer in range(block_tables.shape[0]):
        p, t = used_slots(block_tables[layer], lens)
        used[p, t] = True
    mask = ~used  # [P][16]
    pool.transpose(0, 2, 1, 3)[mask] = BF16_NAN


# ---------------------------------------------------------------------------
# host-resident cases (small enough for the oracle)
# ---------------------------------------------------------------------------

def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(size=shape, dtype=np.float32)
    raise ValueError(dist)


def make_decode_case(name: str, seed: int, lens, num_layers: int = 1, num_pages: Optional[int] = None,
                     max_blocks: Optional[int] = None, dist: str = "normal", layout: str = "random",
                     poison: bool = True, outlier_frac: float = 0.0, outlier_mult: float = 20.0,
                     scale: float = 0.125) -> PagedCase:
    """Host-resident decode case with every tensor drawn from (seed, layer, tensor) streams."""
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    need = pages_needed(lens)
    if max_blocks is None:
        max_blocks = max(int(need.max()), 1)
    if num_pages is None:
        num_pages = max(int(need.sum()) * num_layers + 3, 4)
    lay_rng = _rng(seed, 0, _T_LAYOUT)
    if layout == "random":
        bt = random_block_tables(lay_rng, lens, num_layers, max_blocks, num_pages)
    elif layout == "fragmented":
        bt = fragmented_block_tables(lay_rng, lens, num_layers, max_blocks, num_pages,
                                     history=min(4000, 8 * num_pages))
    else:
        raise ValueError(layout)
    shape_pool = (num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM)
    kp = _draw(_rng(seed, 0, _T_KPOOL), shape_pool, dist)
    vp = _draw(_rng(seed, 0, _T_VPOOL), shape_pool, dist)
    outl = None
    if outlier_frac > 0:
        flat = []
        for layer in range(num_layers):
            p, t = used_slots(bt[layer], lens)
            flat.append(p * PAGE_SIZE + t)
        flat = np.concatenate(flat)
        orng = _rng(seed, 0, _T_OUTLIER)
        outl = np.sort(orng.choice(flat, size=max(1, int(round(outlier_frac * len(flat)))), replace=False))
        pg, sl = outl // PAGE_SIZE, outl % PAGE_SIZE
        kp[pg, :, sl, :] *= outlier_mult
        vp[pg, :, sl, :] *= outlier_mult
    k_pool = f32_to_bf16_bits(kp)
    v_pool = f32_to_bf16_bits(vp)
    del kp, vp
    q = np.stack([f32_to_bf16_bits(_draw(_rng(seed, l, _T_Q), (B, NUM_Q_HEADS, HEAD_DIM), dist))
                  for l in range(num_layers)])
    k_new = np.stack([f32_to_bf16_bits(_draw(_rng(seed, l, _T_KNEW), (B, NUM_KV_HEADS, HEAD_DIM), dist))
                      for l in range(num_layers)])
    v_new = np.stack([f32_to_bf16_bits(_draw(_rng(seed, l, _T_VNEW), (B, NUM_KV_HEADS, HEAD_DIM), dist))
                      for l in range(num_layers)])
    if poison:
        poison_unused(k_pool, bt, lens)
        poison_unused(v_pool, bt, lens)
    return PagedCase(name=name, num_layers=num_layers, num_seqs=B, max_blocks=max_blocks,
                     num_pages=num_pages, context_lens=lens, block_tables=bt, q=q, k_new=k_new,
                     v_new=v_new, k_pool=k_pool, v_pool=v_pool, scale=scale, seed=seed,
                     outlier_slots=outl)


def tiny_decode(seed: int = 0, poison: bool = True) -> PagedCase:
    """1 sequence, 1 layer, 64 tokens on 4 pages at random ids of a 64-page pool, U(-1,1)."""
    return make_decode_case("tiny_decode", seed, [64], num_layers=1, num_pages=64, max_blocks=4,
                            dist="uniform", poison=poison)


def batch8_decode(seed: int = 1, poison: bool = True) -> PagedCase:
    """8 sequences, 1 layer, L ~ U[1, 2048], 4096-page pool (128 MiB of K+V), N(0,1)."""
    lens = _rng(seed, 0, _T_LENS).integers(1, MAX_CONTEXT + 1, size=8).astype(np.int32)
    return make_decode_case("batch8_decode", seed, lens, num_layers=1, num_pages=4096,
                            max_blocks=MAX_CONTEXT // PAGE_SIZE, dist="normal", poison=poison)


def ragged_lengths(seed: int, num_seqs: int) -> np.ndarray:
    """L = clip(rint(exp(N(6, 1))), 1, 2048)."""
    z = _rng(seed, 0, _T_LENS).normal(6.0, 1.0, size=num_seqs)
    return np.clip(np.rint(np.exp(z)), 1, MAX_CONTEXT).astype(np.int32)


# ---------------------------------------------------------------------------
# device-resident cases (full-size configs; pools drawn on the GPU)
# ---------------------------------------------------------------------------

@dataclass
class DeviceCaseSpec:
    """Shape/layout of a full-size multi-layer decode workload.

    The page tables, lengths, q and new-token rows are drawn on the host; the
    pool (GiB-sized) is drawn on the device by :func:`fill_pool_device` from a
    seeded torch generator, in chunks, so nothing of that size visits the host.
    """

    name: str
    num_layers: int
    num_seqs: int
    max_blocks: int
    num_pages: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    seed: int
    outlier_slots: Optional[np.ndarray] = None
    outlier_mult: float = 20.0
    scale: float = 0.125
    theta: float = ROPE_THETA
    extra: dict = field(default_factory=dict)

    def kv_bytes(self) -> int:
        return int(self.context_lens.astype(np.int64).sum()) * KV_BYTES_PER_TOKEN_LAYER * self.num_layers

    def host_rows(self, layer: int):
        """q, k_new, v_new (uint16, pre-RoPE) of one layer, N(0,1)."""
        B = self.num_seqs
        q = f32_to_bf16_bits(_draw(_rng(self.seed, layer, _T_Q), (B, NUM_Q_HEADS, HEAD_DIM), "normal"))
        kn = f32_to_bf16_bits(_draw(_rng(self.seed, layer, _T_KNEW), (B, NUM_KV_HEADS, HEAD_DIM), "normal"))
        vn = f32_to_bf16_bits(_draw(_rng(self.seed, layer, _T_VNEW), (B, NUM_KV_HEADS, HEAD_DIM), "normal"))
        return q, kn, vn


def batch64_spec(seed: int = 2, num_layers: int = 16, num_seqs: int = 64, ctx: int = MAX_CONTEXT) -> DeviceCaseSpec:
    """64 sequences x 2048 tokens (2047 cached + the appended one) x 16 layers.

    Pool sized to fit exactly: 64 x 128 pages x 16 layers = 131072 pages
    (2 GiB of K + 2 GiB of V); page ids are a random permutation over
    (layer, seq, block).
    """
    lens = np.full(num_seqs, ctx, dtype=np.int32)
    mb = (ctx + PAGE_SIZE - 1) // PAGE_SIZE
    num_pages = num_seqs * mb * num_layers
    bt = random_block_tables(_rng(seed, 0, _T_LAYOUT), lens, num_layers, mb, num_pages)
    return DeviceCaseSpec("batch64_decode", num_layers, num_seqs, mb, num_pages, lens, bt, seed)


def batch256_spec(seed: int = 3, num_layers: int = 16, num_seqs: int = 256) -> DeviceCaseSpec:
    """256 ragged sequences (lognormal(6,1) lengths), fragmented pool, 1% outlier rows x20."""
    lens = ragged_lengths(seed, num_seqs)
    need = int(pages_needed(lens).sum()) * num_layers
    num_pages = int(need * 1.25)
    mb = MAX_CONTEXT // PAGE_SIZE
    bt = fragmented_block_tables(_rng(seed, 0, _T_LAYOUT), lens, num_layers, mb, num_pages, history=6000)
    flat = []
    for layer in range(num_layers):
        p, t = used_slots(bt[layer], lens)
        flat.append(p * PAGE_SIZE + t)
    flat = np.concatenate(flat)
    outl = np.sort(_rng(seed, 0, _T_OUTLIER).choice(flat, size=int(round(0.01 * len(flat))), replace=False))
    return DeviceCaseSpec("batch256_ragged", num_layers, num_seqs, mb, num_pages, lens, bt, seed,
                          outlier_slots=outl)


def fill_pool_device(spec: DeviceCaseSpec, device, which: str, chunk_pages: int = 8192, out=None):
    """Draw one pool (``which`` in {"k", "v"}) on the device: N(0,1) -> (x20 outlier rows) -> bf16.
    ``out``: an existing bf16 [num_pages][8][16][64] device tensor to fill instead of a new one."""
    import torch

    tid = _T_KPOOL if which == "k" else _T_VPOOL
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([spec.seed, tid]).generate_state(1)[0]))
    shape = (spec.num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM)
    if out is None:
        pool = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        if tuple(out.shape) != shape or out.dtype != torch.bfloat16:
            raise ValueError(f"out must be bf16 {shape}, got {out.dtype} {tuple(out.shape)}")
        pool = out
    mult = None
    if spec.outlier_slots is not None and len(spec.outlier_slots):
        mult = torch.ones(spec.num_pages * PAGE_SIZE, dtype=torch.float32, device=device)
        mult[torch.from_numpy(spec.outlier_slots).to(device)] = spec.outlier_mult
        mult = mult.view(spec.num_pages, 1, PAGE_SIZE, 1)
    for p0 in range(0, spec.num_pages, chunk_pages):
        p1 = min(spec.num_pages, p0 + chunk_pages)
        x = torch.randn((p1 - p0, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM), dtype=torch.float32, device=device,
                        generator=gen)
        if mult is not None:
            x.mul_(mult[p0:p1])
        pool[p0:p1].copy_(x)
        del x
    return pool


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

def make_prefill_case(name: str, seed: int, prefix_lens, chunk_len: int, num_pages: Optional[int] = None,
                      dist: str = "normal", poison: bool = True, max_blocks: Optional[int] = None) -> PrefillCase:
    prefix = np.asarray(prefix_lens, dtype=np.int32)
    B = len(prefix)
    total = prefix + chunk_len
    need = pages_needed(total)
    if max_blocks is None:
        max_blocks = int(need.max())
    if num_pages is None:
        num_pages = int(need.sum()) + 5
    bt = random_block_tables(_rng(seed, 0, _T_LAYOUT), total, 1, max_blocks, num_pages)[0]
    shape_pool = (num_pages, NUM_KV_HEADS, PAGE_SIZE, HEAD_DIM)
    k_pool = f32_to_bf16_bits(_draw(_rng(seed, 0, _T_KPOOL), shape_pool, dist))
    v_pool = f32_to_bf16_bits(_draw(_rng(seed, 0, _T_VPOOL), shape_pool, dist))
    if poison:
        # the chunk's own slots are overwritten by the append, the prefix must be live
        poison_unused(k_pool, bt[None], total)
        poison_unused(v_pool, bt[None], total)
    q = f32_to_bf16_bits(_draw(_rng(seed, 0, _T_Q), (B, chunk_len, NUM_Q_HEADS, HEAD_DIM), dist))
    kc = f32_to_bf16_bits(_draw(_rng(seed, 0, _T_KNEW), (B, chunk_len, NUM_KV_HEADS, HEAD_DIM), dist))
    vc = f32_to_bf16_bits(_draw(_rng(seed, 0, _T_VNEW), (B, chunk_len, NUM_KV_HEADS, HEAD_DIM), dist))
    return PrefillCase(name=name, num_seqs=B, chunk_len=chunk_len, max_blocks=max_blocks, num_pages=num_pages,
                       prefix_lens=prefix, block_tables=bt, q=q, k_chunk=kc, v_chunk=vc, k_pool=k_pool,
                       v_pool=v_pool, seed=seed)


def prefill_config(seed: int = 4) -> PrefillCase:
    """4 sequences, 1536 cached prefix tokens + a 512-token chunk, 4096-page pool."""
    return make_prefill_case("chunked_prefill", seed, [1536] * 4, 512, num_pages=4096,
                             max_blocks=MAX_CONTEXT // PAGE_SIZE)


# ---------------------------------------------------------------------------
# greedy-decoding logits (argmax)
# ---------------------------------------------------------------------------

VOCAB_SIZE = 128256  # Llama 3.2 vocabulary (tiny-vllm ch.2, "Preallocating the 16 compute buffers")
_T_LOGITS = 20


def argmax_logits(seed: int, rows: int, vocab: int = VOCAB_SIZE, specials: bool = True) -> np.ndarray:
    """Seeded N(0,1) logit rows as float32 [rows][vocab].  With ``specials``, a
    few rows carry the cases a greedy choice must get right: the maximum
    repeated at several places, NaN entries, a -inf row, an all-NaN row and
    signed zeros.  Callers round to bf16 themselves when they need it."""
    rng = _rng(seed, 0, _T_LOGITS)
    x = rng.standard_normal((rows, vocab), dtype=np.float32)
    if specials and rows >= 6 and vocab >= 8:
        x[0, rng.choice(vocab, 4, replace=False)] = 12.0                     # tied maxima
        x[1, rng.choice(vocab, max(1, vocab // 100), replace=False)] = np.nan  # scattered NaN
        x[1, 0] = np.nan
        x[2, :] = -np.inf                                                   # all -inf
        x[2, rng.integers(vocab)] = np.nan
        x[3, :] = np.nan                                                    # only NaN
        x[4, :] = -1.0                                                      # signed zeros tie
        x[4, vocab // 2] = -0.0
        x[4, vocab - 1] = 0.0
        x[5, vocab - 1] = 50.0                                              # maximum at the very end
    return x
