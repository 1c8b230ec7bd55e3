"""Seeded synthetic inputs for paged-attention decode.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests. It only draws random numbers and lays them out (sequence
lengths, block tables, slot mappings, query and key/value source rows, and the
list of cache slots that no sequence references). It holds none of the
attention arithmetic and none of the cache quantisation: the rows it returns
are *sources* that the cache writer (GPU or oracle) turns into a cache.

The five named workloads follow the shapes of the paged-attention problem as
the vLLM-fork pages state it (PagedAttention in the nvllm page's "About"
section; split-K paged decode with an int8 KV cache and a virtual-batch path
for speculative positions in the vllm-sm70 page's "Why" section; 8 target
query tokens per verification step in the vllm-sm12x-nvfp4-dflash2 page's
"What makes this stack different" section; a shared prefix cache in the same
section). Sizes, dtypes and the draw order are fixed here so that both sides
of a parity test see identical bytes:

1. one ``numpy.random.default_rng(seed)`` per workload;
2. sequence lengths: ``rng.integers(lo, hi + 1, size=B)`` for a range, else a
   constant;
3. physical blocks: a fixed pool (``rng.permutation(pool)[:blocks]``) for the
   tiny case, else ``rng.permutation(num_blocks)`` dealt out sequence by
   sequence with ``num_blocks = sum(ceil(L_b / 16)) + 64`` slack blocks; with a
   shared prefix the first ids of the permutation form the prefix blocks that
   every sequence maps;
4. peaked keys: per sequence ``rng.choice(L_b, round(frac * L_b), replace=False)``
   positions whose K rows (all KV heads) are multiplied by a power of two;
5. ``q = rng.standard_normal((B, Tq, Hq, D), float32)``; then per segment in
   logical order (the shared prefix once, then each sequence's private part)
   ``K = standard_normal((n, Hkv, D))`` followed by ``V`` of the same shape;
6. casts to bfloat16 round to nearest even (what ``torch.to(bfloat16)`` does).

Table entries past a sequence's last block, and every slot that no sequence
references, point at / belong to slack blocks that tests fill with poison.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16
SLACK_BLOCKS = 64

DTYPES = ("f32", "bf16", "i8", "fp8", "nvfp4")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even).

    Returns the raw 16-bit patterns as uint16. Input preparation only: the
    generator hands both sides the same bfloat16 source values.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and dtype description of one synthetic decode workload."""

    name: str
    B: int
    Tq: int
    Hq: int
    Hkv: int
    D: int
    seq_lens: Tuple[int, int]  # (lo, hi); lo == hi means constant
    q_dtype: str  # "f32" | "bf16"
    src_dtype: str  # dtype of the K/V source rows handed to the cache writer
    cache_dtype: str  # "f32" | "bf16" | "i8" | "fp8" (OCP E4M3 codes) | "nvfp4"
    pool_blocks: int = 0  # >0: fixed pool size (tiny case); 0: sum of blocks + slack
    peaked_frac: float = 0.0  # fraction of key positions scaled by peak_factor
    peak_factor: float = 8.0
    shared_prefix: int = 0  # tokens whose blocks every sequence shares
    partition_size: int = 0  # split-K partition the workload names (0: heuristic)
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads of the problem statement, at full size.
SPECS: Dict[str, Spec] = {
    "tiny_f32": Spec(
        "tiny_f32", B=1, Tq=1, Hq=4, Hkv=1, D=64, seq_lens=(256, 256),
        q_dtype="f32", src_dtype="f32", cache_dtype="f32", pool_blocks=64,
        description="tiny paged decode: 16 blocks permuted in a 64-block pool, fp32",
    ),
    "gqa_bf16": Spec(
        "gqa_bf16", B=8, Tq=1, Hq=32, Hkv=8, D=128, seq_lens=(1024, 4096),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="bf16",
        description="batched GQA decode, lengths uniform in [1024, 4096], bf16",
    ),
    "long64k_bf16": Spec(
        "long64k_bf16", B=4, Tq=1, Hq=24, Hkv=4, D=256, seq_lens=(65536, 65536),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="bf16", peaked_frac=0.01,
        partition_size=512,
        description="long-context concurrent decode, 64K tokens each, 1% keys x8, bf16",
    ),
    "int8_250k": Spec(
        "int8_250k", B=1, Tq=1, Hq=24, Hkv=4, D=256, seq_lens=(250000, 250000),
        q_dtype="bf16", src_dtype="f32", cache_dtype="i8", partition_size=512,
        description="int8-KV ultra-long decode, 250000 tokens, fp32 N(0,1) source",
    ),
    "verify_bf16": Spec(
        "verify_bf16", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(16384, 32768),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="bf16", shared_prefix=4096,
        description="speculative verify, 8 query tokens, 4096-token shared prefix, bf16 KV",
    ),
    "verify_i8": Spec(
        "verify_i8", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(16384, 32768),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="i8", shared_prefix=4096,
        description="speculative verify, 8 query tokens, 4096-token shared prefix, int8 KV",
    ),
    # FP8 (OCP E4M3) KV variants of the two quantised workloads: same shapes,
    # same seeded draws, the cache writer quantises to FP8 instead of int8
    "fp8_250k": Spec(
        "fp8_250k", B=1, Tq=1, Hq=24, Hkv=4, D=256, seq_lens=(250000, 250000),
        q_dtype="bf16", src_dtype="f32", cache_dtype="fp8",
        description="FP8-KV ultra-long decode, 250000 tokens, fp32 N(0,1) source",
    ),
    "verify_fp8": Spec(
        "verify_fp8", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(16384, 32768),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="fp8", shared_prefix=4096,
        description="speculative verify, 8 query tokens, 4096-token shared prefix, FP8 KV",
    ),
    # NVFP4 KV variants (E2M1 codes, E4M3 scale per 16 elements, fp32 row scale)
    "nvfp4_250k": Spec(
        "nvfp4_250k", B=1, Tq=1, Hq=24, Hkv=4, D=256, seq_lens=(250000, 250000),
        q_dtype="bf16", src_dtype="f32", cache_dtype="nvfp4",
        description="NVFP4-KV ultra-long decode, 250000 tokens, fp32 N(0,1) source",
    ),
    "verify_nvfp4": Spec(
        "verify_nvfp4", B=4, Tq=8, Hq=24, Hkv=4, D=256, seq_lens=(16384, 32768),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="nvfp4", shared_prefix=4096,
        description="speculative verify, 8 query tokens, 4096-token shared prefix, NVFP4 KV",
    ),
    # A batch of decodes that share a long prefix (prefix caching: the
    # vllm-sm12x-nvfp4-dflash2 page's capacity-first profile; the 1Cat-vLLM
    # docs index's feature list): 16 sequences whose first 32768 tokens sit in
    # the same physical blocks, each with 1024..4096 tokens of its own
    "prefix32k_bf16": Spec(
        "prefix32k_bf16", B=16, Tq=1, Hq=24, Hkv=4, D=256, seq_lens=(33792, 36864),
        q_dtype="bf16", src_dtype="bf16", cache_dtype="bf16", shared_prefix=32768,
        description="16 decodes sharing a 32768-token prefix, 1-4K own tokens each, bf16 KV",
    ),
}


@dataclasses.dataclass
class Workload:
    """One generated workload. Arrays are host (numpy) arrays.

    ``q`` is float32 [B, Tq, Hq, D]; when ``spec.q_dtype == "bf16"`` the values
    are already rounded to bfloat16 and ``q_bits`` holds their patterns.
    ``k_src``/``v_src`` are the cache writer's source rows [N, Hkv, D] in the
    source dtype (float32 array, or uint16 bfloat16 patterns), written at
    ``slot_mapping`` [N] (int64; ``slot = block * 16 + offset``).
    """

    spec: Spec
    seed: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks]
    num_blocks: int
    q: np.ndarray  # float32 [B, Tq, Hq, D]
    q_bits: Optional[np.ndarray]  # uint16 when bf16
    k_src: np.ndarray
    v_src: np.ndarray
    slot_mapping: np.ndarray  # int64 [N]
    row_seq: np.ndarray  # int32 [N]: sequence of each source row (-1: shared prefix)
    row_pos: np.ndarray  # int64 [N]: logical position of each source row
    softmax_scale: float  # float32-representable
    slack_blocks: np.ndarray  # int32: blocks no table entry (within a sequence) uses

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def q_array(self) -> np.ndarray:
        """q in its declared dtype: float32, or uint16 bfloat16 patterns."""
        return self.q_bits if self.q_bits is not None else self.q

    def step_rows(self) -> np.ndarray:
        """Indices into the source rows of each sequence's last Tq tokens.

        These are the rows a decode step appends before attending (the query
        tokens' own keys and values).
        """
        out = []
        Tq = self.spec.Tq
        for b in range(self.spec.B):
            L = int(self.seq_lens[b])
            for pos in range(max(L - Tq, 0), L):
                idx = np.nonzero((self.row_seq == b) & (self.row_pos == pos))[0]
                if idx.size:
                    out.append(int(idx[0]))
        return np.asarray(out, dtype=np.int64)

    def unused_slots(self) -> np.ndarray:
        """All cache slots (block * 16 + offset) that hold no source row."""
        used = np.zeros(self.num_blocks * BLOCK_SIZE, dtype=bool)
        used[self.slot_mapping[self.slot_mapping >= 0]] = True
        return np.nonzero(~used)[0].astype(np.int64)


def softmax_scale_for(D: int) -> float:
    """1/sqrt(D) as the float32 value both sides use."""
    return float(np.float32(1.0 / math.sqrt(D)))


def _draw_lengths(rng: np.random.Generator, spec: Spec) -> np.ndarray:
    lo, hi = spec.seq_lens
    if lo == hi:
        return np.full(spec.B, lo, dtype=np.int64)
    return rng.integers(lo, hi + 1, size=spec.B)


def _source(rng: np.random.Generator, n: int, Hkv: int, D: int) -> np.ndarray:
    return rng.standard_normal((n, Hkv, D), dtype=np.float32)


def generate(spec: Spec | str, seed: int = 0, seq_lens: Optional[Sequence[int]] = None) -> Workload:
    """Draw one workload. ``seq_lens`` overrides the drawn lengths (tests)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    bs = BLOCK_SIZE
    rng = np.random.default_rng(seed)
    L = _draw_lengths(rng, spec)
    if seq_lens is not None:
        L = np.asarray(seq_lens, dtype=np.int64)
        assert L.shape == (spec.B,)
    nblk = [(int(x) + bs - 1) // bs for x in L]
    max_len = int(L.max()) if L.size else 0
    max_blocks = max(1, (max_len + bs - 1) // bs)
    P = spec.shared_prefix
    assert P % bs == 0
    if P:
        assert all(int(x) >= P + spec.Tq for x in L), "query tokens must lie past the shared prefix"
    shared_blocks = P // bs

    if spec.pool_blocks:
        assert spec.B == 1 and not P
        num_blocks = spec.pool_blocks
        perm = rng.permutation(num_blocks)
        table_rows = [perm[: nblk[0]]]
    else:
        private = [n - shared_blocks for n in nblk]
        num_blocks = shared_blocks + sum(private) + SLACK_BLOCKS
        perm = rng.permutation(num_blocks)
        prefix_ids = perm[:shared_blocks]
        cursor = shared_blocks
        table_rows = []
        for b in range(spec.B):
            ids = perm[cursor: cursor + private[b]]
            cursor += private[b]
            table_rows.append(np.concatenate([prefix_ids, ids]))
    referenced = np.zeros(num_blocks, dtype=bool)
    for r in table_rows:
        referenced[r] = True
    slack = np.nonzero(~referenced)[0].astype(np.int32)
    assert slack.size > 0
    table = np.empty((spec.B, max_blocks), dtype=np.int32)
    for b in range(spec.B):
        table[b, :] = slack[b % slack.size]  # past-the-end entries point at poisoned blocks
        table[b, : nblk[b]] = table_rows[b]

    peaked: List[np.ndarray] = []
    if spec.peaked_frac > 0:
        for b in range(spec.B):
            peaked.append(rng.choice(int(L[b]), size=int(round(spec.peaked_frac * int(L[b]))), replace=False))

    q = rng.standard_normal((spec.B, spec.Tq, spec.Hq, spec.D), dtype=np.float32)

    ks, vs, seqs, poss = [], [], [], []
    if P:
        ks.append(_source(rng, P, spec.Hkv, spec.D))
        vs.append(_source(rng, P, spec.Hkv, spec.D))
        seqs.append(np.full(P, -1, dtype=np.int32))
        poss.append(np.arange(P, dtype=np.int64))
    for b in range(spec.B):
        n = int(L[b]) - P
        kb = _source(rng, n, spec.Hkv, spec.D)
        vb = _source(rng, n, spec.Hkv, spec.D)
        if peaked:
            sel = peaked[b] - P
            sel = sel[sel >= 0]
            kb[sel] *= np.float32(spec.peak_factor)
        ks.append(kb)
        vs.append(vb)
        seqs.append(np.full(n, b, dtype=np.int32))
        poss.append(np.arange(P, int(L[b]), dtype=np.int64))
    k_src = np.concatenate(ks) if ks else np.zeros((0, spec.Hkv, spec.D), np.float32)
    v_src = np.concatenate(vs) if vs else np.zeros((0, spec.Hkv, spec.D), np.float32)
    row_seq = np.concatenate(seqs) if seqs else np.zeros(0, np.int32)
    row_pos = np.concatenate(poss) if poss else np.zeros(0, np.int64)

    # slot of each source row: its sequence's (or the prefix's) physical block
    slots = np.empty(row_pos.shape[0], dtype=np.int64)
    for b in range(-1 if P else 0, spec.B):
        m = row_seq == b
        pos = row_pos[m]
        tb = table[0] if b < 0 else table[b]
        slots[m] = tb[pos // bs].astype(np.int64) * bs + pos % bs

    q_bits = None
    if spec.q_dtype == "bf16":
        q_bits = bf16_bits(q)
        q = bf16_bits_to_f32(q_bits).reshape(q.shape)
    if spec.src_dtype == "bf16":
        k_src = bf16_bits(k_src).reshape(k_src.shape)
        v_src = bf16_bits(v_src).reshape(v_src.shape)

    return Workload(
        spec=spec, seed=seed, seq_lens=L.astype(np.int32), block_table=table,
        num_blocks=num_blocks, q=q, q_bits=q_bits, k_src=k_src, v_src=v_src,
        slot_mapping=slots, row_seq=row_seq, row_pos=row_pos,
        softmax_scale=softmax_scale_for(spec.D), slack_blocks=slack,
    )


def scaled(spec: Spec | str, **changes) -> Spec:
    """A copy of a named spec with some fields changed (smaller test sizes)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    return dataclasses.replace(spec, **changes)


def kv_bytes_per_token(spec: Spec) -> int:
    """Bytes of K and V (plus int8/FP8 scales) one context token costs per step."""
    if spec.cache_dtype == "nvfp4":
        # codes and block scales (D/2 + D/16 bytes), plus the fp32 row scale
        return 2 * spec.Hkv * (spec.D // 2 + spec.D // 16 + 4)
    elt = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[spec.cache_dtype]
    b = 2 * spec.Hkv * spec.D * elt
    if spec.cache_dtype in ("i8", "fp8"):
        b += 2 * spec.Hkv * 4
    return b
