"""Seeded synthetic inputs for paged varlen attention.

This module only builds inputs: sequence lengths, a shuffled physical block
pool, the per-sequence ``block_table``, the ``slot_mapping`` of the new tokens
and bf16 Q/K/V values.  It holds none of the attention arithmetic, so both the
HIP path and the fp64 oracle can consume what it produces.

Conventions (the KV-cache layout is ``(2, num_blocks, block_size, Hkv, D)``,
K in plane 0 and V in plane 1, as in the FlashAttention backend class
hierarchy of "FlashAttention 在 vLLM 中的实现分析", section 2.1):

* bf16 tensors are held as ``uint16`` bit patterns.  Values are fp32 N(0,1)
  draws rounded to bf16 with round-to-nearest-even.
* Sequence ``b`` has ``Lq_b`` query tokens and ``Lk_b`` keys.  Its query
  tokens are its last ``Lq_b`` positions ``[Lk_b - Lq_b, Lk_b)``; their K/V
  are *new* this step and reach the cache through ``slot_mapping``
  (``slot = block_table[b, p // BS] * BS + p % BS``).  Positions before them
  are already cached.
* Cache slots that hold no valid key (new-token slots before the scatter,
  the slack of each sequence's last block, unused blocks) hold ``SENTINEL``,
  a bf16 quiet NaN, so a missed write or an unmasked read shows up.
* ``block_table`` rows are padded with -1 past ``ceil(Lk_b / BS)``.
* Every random stream is a numpy ``PCG64`` seeded by ``[seed, tag, index]``,
  so one sequence's K/V can be regenerated without building the whole cache.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

SENTINEL = np.uint16(0x7FC1)  # bf16 quiet NaN

# stream tags
_TAG_LEN, _TAG_PERM, _TAG_KV, _TAG_Q, _TAG_PREFIX, _TAG_ORDER, _TAG_SAMPLE = range(7)


def _rng(seed: int, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(tag), int(idx)]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite normal draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def randn_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclasses.dataclass
class Spec:
    """Shape of one synthetic batch (before any random draw)."""
    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    causal: bool
    seed: int
    # list of ("decode"|"prefill", lo, hi): lengths drawn uniform in [lo, hi]
    groups: Tuple[Tuple[str, int, int, int], ...] = ()   # (kind, count, lo, hi)
    fixed: Optional[Tuple[Tuple[int, int], ...]] = None   # explicit (Lq, Lk)
    min_num_blocks: int = 0
    shared_prefix: int = 0          # tokens shared at the head of every sequence
    shuffle_order: bool = False     # interleave groups in a seeded order
    description: str = ""


SPECS = {
    "tiny_mixed": Spec(
        name="tiny_mixed", num_heads=4, num_kv_heads=2, head_size=64, block_size=16,
        causal=True, seed=1001, fixed=((37, 37), (1, 81)), min_num_blocks=16,
        description="2 seqs: 37-token causal prefill + 1-token decode over 80 cached "
                    "tokens; H=4 Hkv=2 D=64 BS=16, 16 physical blocks"),
    "decode_llama8b": Spec(
        name="decode_llama8b", num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
        causal=True, seed=1002, groups=(("decode", 64, 512, 4096),),
        description="64 decode seqs, Lk~U[512,4096]; H=32 Hkv=8 D=128 BS=16"),
    "chunked_prefill_mix": Spec(
        name="chunked_prefill_mix", num_heads=32, num_kv_heads=8, head_size=128,
        block_size=32, causal=True, seed=1003,
        groups=(("prefill", 8, 256, 2048), ("decode", 56, 256, 4096)), shuffle_order=True,
        description="8 causal prefills L~U[256,2048] + 56 decodes Lk~U[256,4096]; "
                    "H=32 Hkv=8 D=128 BS=32, one launch"),
    "chunked_prefill_mix_prefill": Spec(
        name="chunked_prefill_mix_prefill", num_heads=32, num_kv_heads=8, head_size=128,
        block_size=32, causal=True, seed=1003, groups=(("prefill", 8, 256, 2048),),
        description="the 8 causal prefills of chunked_prefill_mix alone (the same seed draws "
                    "the same lengths first); H=32 Hkv=8 D=128 BS=32"),
    "prefill_causal_8k": Spec(
        name="prefill_causal_8k", num_heads=32, num_kv_heads=8, head_size=128, block_size=32,
        causal=True, seed=1010, groups=(("prefill", 4, 8192, 8192),),
        description="4 causal prefills of 8192 tokens; H=32 Hkv=8 D=128 BS=32 (long-prefill "
                    "counterpart of chunked_prefill_mix_prefill)"),
    "cascade_prefix": Spec(
        name="cascade_prefix", num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
        causal=True, seed=1004, groups=(("decode", 32, 64, 512),), shared_prefix=2048,
        description="32 decode reqs sharing a 2048-token prefix + private suffix "
                    "U[64,512]; H=32 Hkv=8 D=128 BS=16"),
    "cascade_prefix_16k": Spec(
        name="cascade_prefix_16k", num_heads=32, num_kv_heads=8, head_size=128, block_size=16,
        causal=True, seed=1006, groups=(("decode", 64, 64, 512),), shared_prefix=16384,
        description="64 decode reqs sharing a 16384-token prefix + private suffix U[64,512]; "
                    "H=32 Hkv=8 D=128 BS=16 (the cascade decision's other side)"),
    "long_decode_d256": Spec(
        name="long_decode_d256", num_heads=16, num_kv_heads=2, head_size=256, block_size=64,
        causal=True, seed=1005, groups=(("decode", 16, 32768, 131072),),
        description="16 decode seqs, Lk~U[32768,131072]; H=16 Hkv=2 (GQA 8) D=256 BS=64"),
}
ORDER = ["tiny_mixed", "decode_llama8b", "chunked_prefill_mix", "cascade_prefix",
         "long_decode_d256"]


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    q_lens: np.ndarray          # int32 [B]
    k_lens: np.ndarray          # int32 [B]  (seqused_k)
    cu_seqlens_q: np.ndarray    # int32 [B+1]
    block_table: np.ndarray     # int32 [B, max_blocks], -1 padded
    num_blocks: int
    slot_mapping: np.ndarray    # int64 [T]
    scale: np.float32
    # bf16 bit patterns; None until materialise() is called
    q: Optional[np.ndarray] = None        # [T, H, D]
    key: Optional[np.ndarray] = None      # [T, Hkv, D]  new tokens
    value: Optional[np.ndarray] = None    # [T, Hkv, D]
    kv_cache: Optional[np.ndarray] = None  # [2, NB, BS, Hkv, D] before the scatter

    @property
    def B(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def H(self) -> int:
        return self.spec.num_heads

    @property
    def Hkv(self) -> int:
        return self.spec.num_kv_heads

    @property
    def D(self) -> int:
        return self.spec.head_size

    @property
    def BS(self) -> int:
        return self.spec.block_size

    @property
    def causal(self) -> bool:
        return self.spec.causal

    def kv_read_bytes(self) -> int:
        """Algorithmic KV bytes of one attention pass: every visible K and V
        element read once, bf16."""
        return int(2 * self.k_lens.astype(np.int64).sum() * self.Hkv * self.D * 2)

    def causal_pairs(self) -> np.ndarray:
        """Unmasked (query, key) pairs per sequence, bottom-right causal."""
        out = np.zeros(self.B, dtype=np.int64)
        for b in range(self.B):
            lq, lk = int(self.q_lens[b]), int(self.k_lens[b])
            if not self.causal:
                out[b] = lq * lk
                continue
            off = lk - lq
            i = np.arange(lq, dtype=np.int64)
            out[b] = np.clip(i + off + 1, 0, lk).sum()
        return out

    def attention_flops(self) -> int:
        """4*D*H flops per unmasked pair (QK^T and PV, 2 flops per MAC)."""
        return int(4 * self.D * self.H * self.causal_pairs().sum())

    def summary(self) -> dict:
        return {"workload": self.spec.name, "batch": self.B, "num_tokens": self.T,
                "num_heads": self.H, "num_kv_heads": self.Hkv, "head_size": self.D,
                "block_size": self.BS, "num_blocks": self.num_blocks,
                "causal": self.causal, "seed": self.seed,
                "sum_k_lens": int(self.k_lens.sum()),
                "max_k_len": int(self.k_lens.max()) if self.B else 0,
                "max_q_len": int(self.q_lens.max()) if self.B else 0}


def _draw_lengths(spec: Spec, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    if spec.fixed is not None:
        q = np.array([a for a, _ in spec.fixed], dtype=np.int32)
        k = np.array([b for _, b in spec.fixed], dtype=np.int32)
        return q, k
    rng = _rng(seed, _TAG_LEN)
    qs: List[int] = []
    ks: List[int] = []
    for kind, count, lo, hi in spec.groups:
        # integers uniform in [lo, hi], both ends included
        lens = rng.integers(lo, hi + 1, size=count)
        for L in lens:
            L = int(L)
            if kind == "decode":
                qs.append(1)
                ks.append(L + spec.shared_prefix)
            elif kind == "prefill":
                qs.append(L)
                ks.append(L + spec.shared_prefix)
            else:
                raise ValueError(kind)
    q = np.array(qs, dtype=np.int32)
    k = np.array(ks, dtype=np.int32)
    if spec.shuffle_order:
        perm = _rng(seed, _TAG_ORDER).permutation(len(q))
        q, k = q[perm], k[perm]
    return q, k


def _allocate_blocks(spec: Spec, seed: int, k_lens: np.ndarray):
    BS = spec.block_size
    B = len(k_lens)
    P = spec.shared_prefix
    if P % BS:
        raise ValueError("shared prefix must be block aligned")
    n_shared = P // BS
    nblk = [(int(L) + BS - 1) // BS for L in k_lens]
    private = [n - n_shared for n in nblk]
    needed = n_shared + sum(private)
    NB = max(needed, spec.min_num_blocks)
    perm = _rng(seed, _TAG_PERM).permutation(NB).astype(np.int32)
    max_blocks = max(nblk) if B else 1
    bt = np.full((B, max(max_blocks, 1)), -1, dtype=np.int32)
    cursor = n_shared
    shared_ids = perm[:n_shared]
    for b in range(B):
        bt[b, :n_shared] = shared_ids
        bt[b, n_shared:nblk[b]] = perm[cursor:cursor + private[b]]
        cursor += private[b]
    return bt, NB


def make(name_or_spec, seed: Optional[int] = None, materialise: bool = True) -> Workload:
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    seed = spec.seed if seed is None else int(seed)
    q_lens, k_lens = _draw_lengths(spec, seed)
    if np.any(q_lens > k_lens):
        raise ValueError("every query token must have its own key")
    bt, NB = _allocate_blocks(spec, seed, k_lens)
    cu = np.zeros(len(q_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    BS = spec.block_size
    slots = []
    for b in range(len(q_lens)):
        p = np.arange(k_lens[b] - q_lens[b], k_lens[b], dtype=np.int64)
        slots.append(bt[b, p // BS].astype(np.int64) * BS + p % BS)
    slot_mapping = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    scale = np.float32(1.0 / math.sqrt(spec.head_size))
    wl = Workload(spec=spec, seed=seed, q_lens=q_lens, k_lens=k_lens, cu_seqlens_q=cu,
                  block_table=bt, num_blocks=NB, slot_mapping=slot_mapping, scale=scale)
    if materialise:
        materialise_values(wl)
    return wl


def sequence_kv(wl: Workload, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows [Lk_b, Hkv, D] (bf16 bits) of sequence b in token order.

    The shared prefix (if any) comes from one stream used by every sequence;
    the rest from the sequence's own stream."""
    spec, seed = wl.spec, wl.seed
    Hkv, D, P = spec.num_kv_heads, spec.head_size, spec.shared_prefix
    Lk = int(wl.k_lens[b])
    parts_k, parts_v = [], []
    if P:
        r = _rng(seed, _TAG_PREFIX)
        parts_k.append(randn_bf16(r, (P, Hkv, D)))
        parts_v.append(randn_bf16(r, (P, Hkv, D)))
    r = _rng(seed, _TAG_KV, b)
    parts_k.append(randn_bf16(r, (Lk - P, Hkv, D)))
    parts_v.append(randn_bf16(r, (Lk - P, Hkv, D)))
    return np.concatenate(parts_k), np.concatenate(parts_v)


def sequence_q(wl: Workload, b: int) -> np.ndarray:
    Lq = int(wl.q_lens[b])
    return randn_bf16(_rng(wl.seed, _TAG_Q, b), (Lq, wl.H, wl.D))


def materialise_values(wl: Workload, only: Optional[Sequence[int]] = None) -> Workload:
    """Fill q, key, value and the pre-scatter cache.

    With ``only`` given, just those sequences' values are drawn (others stay
    SENTINEL / zero) so a sample of a large batch can be rebuilt cheaply."""
    H, Hkv, D, BS = wl.H, wl.Hkv, wl.D, wl.BS
    T = wl.T
    q = np.zeros((T, H, D), dtype=np.uint16)
    key = np.full((T, Hkv, D), SENTINEL, dtype=np.uint16)
    value = np.full((T, Hkv, D), SENTINEL, dtype=np.uint16)
    cache = np.full((2, wl.num_blocks, BS, Hkv, D), SENTINEL, dtype=np.uint16)
    seqs = range(wl.B) if only is None else only
    for b in seqs:
        Lq, Lk = int(wl.q_lens[b]), int(wl.k_lens[b])
        t0 = int(wl.cu_seqlens_q[b])
        Kb, Vb = sequence_kv(wl, b)
        q[t0:t0 + Lq] = sequence_q(wl, b)
        key[t0:t0 + Lq] = Kb[Lk - Lq:]
        value[t0:t0 + Lq] = Vb[Lk - Lq:]
        n_cached = Lk - Lq
        nfull = (n_cached + BS - 1) // BS
        if nfull:
            padK = np.full((nfull * BS, Hkv, D), SENTINEL, dtype=np.uint16)
            padV = padK.copy()
            padK[:n_cached] = Kb[:n_cached]
            padV[:n_cached] = Vb[:n_cached]
            ids = wl.block_table[b, :nfull]
            # the last partially cached block also holds new-token slots:
            # those stay SENTINEL until the scatter writes them
            cache[0, ids] = padK.reshape(nfull, BS, Hkv, D)
            cache[1, ids] = padV.reshape(nfull, BS, Hkv, D)
    wl.q, wl.key, wl.value, wl.kv_cache = q, key, value, cache
    return wl


def sample_sequences(wl: Workload, n: int) -> List[int]:
    """A seeded choice of n distinct sequence indices (sorted)."""
    n = min(n, wl.B)
    return sorted(int(i) for i in _rng(wl.seed, _TAG_SAMPLE).choice(wl.B, size=n, replace=False))


def to_device(wl: Workload, device="cuda") -> dict:
    """Torch tensors of a materialised workload (bf16 via a bit-preserving
    view of the uint16 patterns)."""
    import torch

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return {
        "q": bf16(wl.q), "key": bf16(wl.key), "value": bf16(wl.value),
        "kv_cache": bf16(wl.kv_cache),
        "slot_mapping": torch.from_numpy(np.ascontiguousarray(wl.slot_mapping, dtype=np.int64)).to(device),
        "cu_seqlens_q": i32(wl.cu_seqlens_q), "seqused_k": i32(wl.k_lens),
        "block_table": i32(wl.block_table),
    }


def fp8_cache_codes(wl: Workload, seed: int) -> np.ndarray:
    """A uint8 (E4M3) cache of the workload's shape: every slot that holds a
    value in the bf16 cache gets a random code of magnitude 0x00..0x57
    (|value| <= 15) and a random sign; every SENTINEL slot gets the NaN code
    0x7F, so that a read of a slot outside the keys shows up as NaN."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 0x58, size=wl.kv_cache.shape, dtype=np.uint8)
    codes |= (rng.integers(0, 2, size=wl.kv_cache.shape, dtype=np.uint8) << 7).astype(np.uint8)
    codes[wl.kv_cache == SENTINEL] = 0x7F
    return codes


def fp8_scales(num_kv_heads: int, seed: int):
    """Per-KV-head fp32 (k_scale, v_scale), uniform in [0.02, 0.1]."""
    rng = np.random.default_rng(seed)
    return (rng.uniform(0.02, 0.1, num_kv_heads).astype(np.float32),
            rng.uniform(0.02, 0.1, num_kv_heads).astype(np.float32))


def bf16_tensor_bits(t) -> np.ndarray:
    """Device/host bf16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
