"""Seeded synthetic inputs for the paged-KV decode path.

Shared by the tests and the benchmark, and by nothing else.  This module holds
none of the method's arithmetic: it draws context lengths, the pool's initial
free-list order and the q / K / V values, and it rounds fp32 draws to the bf16
input dtype.  Block tables, slots and copy pairs are produced by an allocator
(the oracle's or the library's) from what is drawn here.

Workloads (all values N(0, 1); bf16 carried as uint16 bit patterns):

  1  tiny       4 seqs, 4 q / 4 kv heads, head_dim 64, block 16, fp32,
                context U{1..64}, 32 physical blocks, scale 1/8
  2  llama8b    64 seqs, 32 q / 8 kv heads, head_dim 128, bf16, block 16,
                context U{128..4096}, pool = ceil(1.25 x blocks needed)
  3  sampling   16 prompts x 8 samples, prompt 2048 - U{1..15} tokens, each
                sample then generates U{1..256} tokens (round-robin steps),
                heads as 2, pool = ceil(1.25 x blocks needed)
  4  longctx    8 seqs x 32768 tokens, heads as 2, partition 512,
                pool = 1.25 x blocks needed (20480)
  5  mixed      256 seqs, context floor(exp(U(ln 16, ln 8192))) clipped to
                [16, 8192], 64 q / 8 kv heads, head_dim 128, bf16,
                block size 8, 16 or 32, one step of 256 appended tokens
  6  prefix     64 requests = one 1024-token system prompt + U{16..1024}
                own tokens (token ids from a 32000-id vocabulary), heads as 2
  7  prefill    16 seqs = cached prefix U{0..2048} + a 512-token chunk of
                new tokens, heads as 2

Random draws come from numpy's PCG64 generator seeded with 1000 + workload
number, in this order: context lengths, free-list permutation, q, K pool, V
pool, new-token k, new-token v.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)


def seed_for(workload: int) -> int:
    return 1000 + workload


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values (finite) to bf16, nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) draws in the input dtype ('bf16' -> uint16 bits, 'f32')."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        return bf16_from_f32(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def nan_bits(dtype: str):
    return BF16_NAN if dtype == "bf16" else np.float32(np.nan)


def np_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


@dataclass
class Shape:
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    scale: float
    partition_size: int = 512

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


SHAPES = {
    1: Shape(4, 4, 4, 64, 16, "f32", 1.0 / 8.0, 512),
    2: Shape(64, 32, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
    3: Shape(128, 32, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
    4: Shape(8, 32, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
    5: Shape(256, 64, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
    6: Shape(64, 32, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
    7: Shape(16, 32, 8, 128, 16, "bf16", 1.0 / math.sqrt(128), 512),
}


def shape(workload: int, block_size: Optional[int] = None) -> Shape:
    s = SHAPES[workload]
    if block_size is None:
        return Shape(**s.__dict__)
    d = dict(s.__dict__)
    d["block_size"] = block_size
    return Shape(**d)


def draw_context_lens(workload: int, rng: np.random.Generator, num_seqs: int) -> np.ndarray:
    if workload == 1:
        return rng.integers(1, 64, size=num_seqs, endpoint=True).astype(np.int32)
    if workload == 2:
        return rng.integers(128, 4096, size=num_seqs, endpoint=True).astype(np.int32)
    if workload == 4:
        return np.full(num_seqs, 32768, dtype=np.int32)
    if workload == 5:
        u = rng.uniform(math.log(16), math.log(8192), size=num_seqs)
        return np.clip(np.floor(np.exp(u)), 16, 8192).astype(np.int32)
    raise ValueError(f"workload {workload} has no plain context-length draw")


def pool_blocks(ctx: np.ndarray, block_size: int, factor: float = 1.25) -> int:
    need = int(sum(-(-int(n) // block_size) for n in ctx))
    return max(1, int(math.ceil(factor * need)))


@dataclass
class DecodeInputs:
    """Everything a decode workload needs except the allocator's output."""
    workload: int
    shape: Shape
    context_lens: np.ndarray          # [S] int32 (tokens per sequence at decode)
    num_blocks: int
    free_order: np.ndarray            # [NB] int32 permutation
    q: np.ndarray                     # [S, Hq, D]
    k_cache: np.ndarray               # [NB, Hkv, B, D]
    v_cache: np.ndarray
    extra: dict = field(default_factory=dict)


def decode_inputs(workload: int, block_size: Optional[int] = None,
                  seed: Optional[int] = None, num_seqs: Optional[int] = None,
                  fill_pool: bool = True) -> DecodeInputs:
    """Draw a decode workload (1, 2, 4).  The pool is filled with N(0,1)
    values everywhere; the allocator decides which blocks are live."""
    sh = shape(workload, block_size)
    if num_seqs is not None:
        sh.num_seqs = num_seqs
    rng = np.random.default_rng(seed_for(workload) if seed is None else seed)
    ctx = draw_context_lens(workload, rng, sh.num_seqs)
    if workload == 1:
        nb = 32
    elif workload == 4:
        nb = pool_blocks(ctx, sh.block_size)
    else:
        nb = pool_blocks(ctx, sh.block_size)
    order = rng.permutation(nb).astype(np.int32)
    q = normal(rng, (sh.num_seqs, sh.num_q_heads, sh.head_dim), sh.dtype)
    pool_shape = (nb, sh.num_kv_heads, sh.block_size, sh.head_dim)
    if fill_pool:
        kc = normal(rng, pool_shape, sh.dtype)
        vc = normal(rng, pool_shape, sh.dtype)
    else:
        kc = np.zeros(pool_shape, dtype=np_dtype(sh.dtype))
        vc = np.zeros(pool_shape, dtype=np_dtype(sh.dtype))
    return DecodeInputs(workload, sh, ctx, nb, order, q, kc, vc)


def mixed_step_inputs(block_size: int, seed: Optional[int] = None,
                      num_seqs: Optional[int] = None) -> DecodeInputs:
    """Workload 5: per-token logical K/V shared by every block size.

    ``extra`` holds 'prefix_k' / 'prefix_v' ([sum(ctx-1), Hkv, D], the tokens
    already in the cache, sequence-major) and 'new_k' / 'new_v' ([S, Hkv, D],
    the tokens the step appends).  The pool arrays are left zero: the caller
    writes the prefix through the allocator's slots.
    """
    sh = shape(5, block_size)
    if num_seqs is not None:
        sh.num_seqs = num_seqs
    rng = np.random.default_rng(seed_for(5) if seed is None else seed)
    ctx = draw_context_lens(5, rng, sh.num_seqs)
    # The pool is sized for the largest block size so every sweep point sees
    # the same permutation draw; block counts differ with B.
    nb = pool_blocks(ctx, block_size)
    order = rng.permutation(nb).astype(np.int32)
    q = normal(rng, (sh.num_seqs, sh.num_q_heads, sh.head_dim), sh.dtype)
    n_prefix = int((ctx - 1).sum())
    pk = normal(rng, (n_prefix, sh.num_kv_heads, sh.head_dim), sh.dtype)
    pv = normal(rng, (n_prefix, sh.num_kv_heads, sh.head_dim), sh.dtype)
    nk = normal(rng, (sh.num_seqs, sh.num_kv_heads, sh.head_dim), sh.dtype)
    nv = normal(rng, (sh.num_seqs, sh.num_kv_heads, sh.head_dim), sh.dtype)
    pool_shape = (nb, sh.num_kv_heads, sh.block_size, sh.head_dim)
    kc = np.zeros(pool_shape, dtype=np_dtype(sh.dtype))
    vc = np.zeros(pool_shape, dtype=np_dtype(sh.dtype))
    return DecodeInputs(5, sh, ctx, nb, order, q, kc, vc,
                        extra={"prefix_k": pk, "prefix_v": pv, "new_k": nk, "new_v": nv})


@dataclass
class SamplingPlan:
    """Workload 3: prompts, samples per prompt and per-sample generation."""
    shape: Shape
    prompt_lens: np.ndarray           # [P] int32
    samples: int
    gen_lens: np.ndarray              # [P * samples] int32, sample-major per prompt
    num_blocks: int
    free_order: np.ndarray


def sampling_plan(seed: Optional[int] = None, num_prompts: int = 16, samples: int = 8,
                  prompt_base: int = 2048, max_gen: int = 256) -> SamplingPlan:
    sh = shape(3)
    sh.num_seqs = num_prompts * samples
    rng = np.random.default_rng(seed_for(3) if seed is None else seed)
    prompt = (prompt_base - rng.integers(1, 15, size=num_prompts, endpoint=True)).astype(np.int32)
    gen = rng.integers(1, max_gen, size=num_prompts * samples, endpoint=True).astype(np.int32)
    B = sh.block_size
    need = 0
    for p in range(num_prompts):
        need += -(-int(prompt[p]) // B)
        for j in range(samples):
            total = int(prompt[p]) + int(gen[p * samples + j])
            # blocks a sample owns beyond the shared prompt blocks (upper bound)
            need += -(-total // B) - int(prompt[p]) // B
    nb = int(math.ceil(1.25 * need))
    order = rng.permutation(nb).astype(np.int32)
    return SamplingPlan(sh, prompt, samples, gen, nb, order)


def poison_unused(k_cache: np.ndarray, v_cache: np.ndarray, tables, context_lens,
                  block_size: int, dtype: str) -> None:
    """Put NaN in every slot no sequence reads: positions >= its length in its
    last block, and every block no table reaches.  In place."""
    nan = nan_bits(dtype)
    nb = k_cache.shape[0]
    live = np.zeros((nb, block_size), dtype=bool)
    for t, n in zip(tables, context_lens):
        n = int(n)
        for i in range(-(-n // block_size)):
            live[int(t[i]), : min(block_size, n - i * block_size)] = True
    dead = ~live  # [NB, B]
    kb = k_cache.transpose(0, 2, 1, 3)  # [NB, B, H, D] view
    vb = v_cache.transpose(0, 2, 1, 3)
    kb[dead] = nan
    vb[dead] = nan


def sampling_ops(plan: SamplingPlan):
    """The operation stream of workload 3, as plain tuples (no arithmetic of the
    method: which sequence to admit, fork or step, in which order).

      ("add", seq, n)          admit sample 0 of a prompt with its n prompt tokens
      ("fork", parent, child)  samples 1 .. samples-1 start as copies of sample 0
      ("step", [seqs])         one generation step of every still-generating
                               sample, in increasing id order (round-robin)

    Sequence id of sample j of prompt p is p * samples + j.
    """
    S = plan.samples
    P = len(plan.prompt_lens)
    for p in range(P):
        yield ("add", p * S, int(plan.prompt_lens[p]))
        for j in range(1, S):
            yield ("fork", p * S, p * S + j)
    for i in range(int(plan.gen_lens.max())):
        active = [s for s in range(P * S) if int(plan.gen_lens[s]) > i]
        yield ("step", active)


@dataclass
class PrefixPlan:
    """Prefix-cache workload: requests that open with one shared system prompt
    (page 3, section 04: a repeated system prompt, then each user's own
    question).  Token ids are labels drawn uniformly from a 32000-id vocabulary."""
    shape: Shape
    system: np.ndarray                # [system_len] int32
    suffixes: List[np.ndarray]        # per request, [suffix_len] int32
    num_blocks: int
    free_order: np.ndarray

    def prompt(self, r: int) -> np.ndarray:
        return np.concatenate([self.system, self.suffixes[r]]).astype(np.int32)


def prefix_plan(seed: Optional[int] = None, num_requests: int = 64, system_len: int = 1024,
                suffix_min: int = 16, suffix_max: int = 1024, vocab: int = 32000,
                spare_blocks: int = 0) -> PrefixPlan:
    """64 requests = a 1024-token system prompt + a suffix of U{16..1024} tokens,
    Llama-3-8B layer shape; the pool is 1.25x the blocks the prompts need with
    sharing, plus ``spare_blocks``, in a seeded random order."""
    sh = shape(6)
    sh.num_seqs = num_requests
    rng = np.random.default_rng(seed_for(6) if seed is None else seed)
    system = rng.integers(0, vocab, size=system_len).astype(np.int32)
    lens = rng.integers(suffix_min, suffix_max, size=num_requests, endpoint=True)
    suffixes = [rng.integers(0, vocab, size=int(n)).astype(np.int32) for n in lens]
    B = sh.block_size
    need = -(-system_len // B) + sum(-(-int(n) // B) + 1 for n in lens)
    nb = int(math.ceil(1.25 * need)) + spare_blocks
    order = rng.permutation(nb).astype(np.int32)
    return PrefixPlan(sh, system, suffixes, nb, order)


@dataclass
class PrefillInputs:
    """Chunked-prefill workload: every sequence has a cached prefix and a
    chunk of new tokens whose K/V are already in the pool (placement of the
    tokens in blocks is left to an allocator, from ``free_order``)."""
    shape: Shape
    context_lens: np.ndarray          # [S] int32, prefix + chunk
    qsl: np.ndarray                   # [S + 1] int32, query_start_loc
    num_blocks: int
    free_order: np.ndarray
    q: np.ndarray                     # [T, Hq, D]
    k_cache: np.ndarray               # [NB, Hkv, B, D]
    v_cache: np.ndarray


def prefill_inputs(seed: Optional[int] = None, num_seqs: int = 16, chunk: int = 512,
                   max_prefix: int = 2048, block_size: int = 16) -> PrefillInputs:
    """16 sequences = a cached prefix of U{0..2048} tokens + a 512-token chunk,
    Llama-3-8B layer shape; a pool 1.25x the blocks needed, its free order a
    seeded permutation."""
    sh = shape(7, block_size)
    sh.num_seqs = num_seqs
    rng = np.random.default_rng(seed_for(7) if seed is None else seed)
    prefix = rng.integers(0, max_prefix, size=num_seqs, endpoint=True)
    ctx = (prefix + chunk).astype(np.int32)
    B = sh.block_size
    need = int(sum(-(-int(n) // B) for n in ctx))
    nb = int(math.ceil(1.25 * need))
    order = rng.permutation(nb).astype(np.int32)
    q = normal(rng, (num_seqs * chunk, sh.num_q_heads, sh.head_dim), sh.dtype)
    kc = normal(rng, (nb, sh.num_kv_heads, B, sh.head_dim), sh.dtype)
    vc = normal(rng, (nb, sh.num_kv_heads, B, sh.head_dim), sh.dtype)
    qsl = np.arange(num_seqs + 1, dtype=np.int32) * chunk
    return PrefillInputs(sh, ctx, qsl, nb, order, q, kc, vc)
