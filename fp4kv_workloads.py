"""Seeded synthetic inputs for the FP4 KV-cache path.

This module only draws random numbers and builds page tables and slot
numbers; it holds none of the quantisation or attention arithmetic.  Both the
HIP path (through the tests and the benchmark) and the CPU oracle are fed from
it, so they see identical bf16 bits.

Recipe: values are drawn as N(0, 1) in fp32 with torch's CPU generator,
multiplied in fp32 by a per-(KV head, channel) factor, and rounded once to
bf16 (round to nearest even).  Every (sequence, tensor, token chunk) has its
own seed, so any slice of a large workload can be regenerated on its own.

The workloads follow the shapes the pages discuss for a decode-bound KV cache
("KV Cache Quantisation", Notes and Common questions: long context, large
batch, paged caches): a tiny single step with an outlier key channel (the
outlier lesson of "Week 6 -- FP4 KV Caches and Bounded Replay", Core
Concepts), GQA batches at 4K and 32K context, one 512K-token sequence, a
mixed-length paged batch, and a prefill.
"""
from dataclasses import dataclass, field
import math
from typing import Dict, List, Optional, Tuple

import torch

PAGE_SIZE = 64          # tokens per cache page
CHUNK_TOKENS = 4096     # seeding granularity along a sequence


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                      # "decode" (contiguous), "paged" or "prefill"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    context: int = 0               # tokens per sequence (decode, prefill)
    splits: int = 0                # split-K chunks; 0 lets the library choose
    min_len: int = 0               # paged: lengths uniform in [min_len, max_len]
    max_len: int = 0
    key_outlier: str = "none"      # how key channels are scaled (see channel_factors)
    value_outlier: str = "none"
    description: str = ""

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def pages_per_seq(self) -> int:
        return -(-self.context // PAGE_SIZE)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_d64_ctx256", "decode", batch=1, q_heads=4, kv_heads=1, head_dim=64,
             context=256, key_outlier="ch7x20",
             description="one step, B 1, Hq 4, Hkv 1, D 64, 256 tokens, key channel 7 x20"),
    Workload("gqa4_b8_ctx4k", "decode", batch=8, q_heads=32, kv_heads=8, head_dim=128,
             context=4096, key_outlier="4chx10",
             description="B 8, Hq 32, Hkv 8, D 128, 4096 tokens, 4 key channels per head x10"),
    Workload("gqa8_b32_ctx32k", "decode", batch=32, q_heads=64, kv_heads=8, head_dim=128,
             context=32768, splits=64, key_outlier="loguniform", value_outlier="loguniform",
             description="B 32, Hq 64, Hkv 8, D 128, 32768 tokens, 64 splits, "
                         "channel std log-uniform in [0.5, 4]"),
    Workload("gqa4_b1_ctx512k", "decode", batch=1, q_heads=32, kv_heads=8, head_dim=128,
             context=524288, splits=256, key_outlier="2chx20",
             description="B 1, Hq 32, Hkv 8, D 128, 524288 tokens, 256 splits, "
                         "2 key channels per head x20"),
    Workload("paged_b64_len1k_16k", "paged", batch=64, q_heads=32, kv_heads=8, head_dim=128,
             min_len=1024, max_len=16384,
             description="B 64, Hq 32, Hkv 8, D 128, lengths uniform in [1024, 16384], "
                         "64-token pages in a seeded random order, append one token then attend"),
    Workload("prefill_b8_8k", "prefill", batch=8, q_heads=32, kv_heads=8, head_dim=128,
             context=8192,
             description="quantise-append of 8 x 8192 tokens, Hkv 8, D 128"),
]}


def _mix(*parts: int) -> int:
    """A 63-bit seed from integers (splitmix64 finaliser over a running hash)."""
    h = 0x9E3779B97F4A7C15
    for p in parts:
        h = (h ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h = (h * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 31
        h = (h * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    return h & 0x7FFFFFFFFFFFFFFF


def _gen(*parts: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(_mix(*parts))
    return g


_TENSOR_ID = {"k": 1, "v": 2, "q": 3, "len": 4, "perm": 5, "factor_k": 6, "factor_v": 7}


def _name_id(name: str) -> int:
    return sum((i + 1) * ord(c) for i, c in enumerate(name))


def channel_factors(w: Workload, seed: int, tensor: str) -> torch.Tensor:
    """fp32 [Hkv][D] multipliers applied to the N(0, 1) draws of K or V."""
    f = torch.ones(w.kv_heads, w.head_dim, dtype=torch.float32)
    kind = w.key_outlier if tensor == "k" else w.value_outlier
    g = _gen(seed, _name_id(w.name), _TENSOR_ID["factor_" + tensor])
    if kind == "ch7x20":
        f[:, 7] = 20.0
    elif kind in ("4chx10", "2chx20"):
        n, mult = (4, 10.0) if kind == "4chx10" else (2, 20.0)
        for h in range(w.kv_heads):
            ch = torch.randperm(w.head_dim, generator=g)[:n]
            f[h, ch] = mult
    elif kind == "loguniform":
        u = torch.rand(w.kv_heads, w.head_dim, generator=g, dtype=torch.float32)
        f = torch.exp(math.log(0.5) + u * (math.log(4.0) - math.log(0.5)))
    elif kind != "none":
        raise ValueError(kind)
    return f


def fp8_tensor_scales(w: Workload, seed: int) -> Tuple[float, float]:
    """(k_scale, v_scale) for an FP8 cache of this workload: the per-tensor
    scale is an input of that format, fixed before any token is stored (as a
    calibrated scale would be).  Chosen here as 6 x the largest channel
    factor of the tensor over 448, so that a 6-sigma value of the widest
    channel maps to the top of the E4M3 range; rounded to fp32."""
    import numpy as np
    ks = np.float32(6.0 * float(channel_factors(w, seed, "k").max()) / 448.0)
    vs = np.float32(6.0 * float(channel_factors(w, seed, "v").max()) / 448.0)
    return float(ks), float(vs)


def kv_tokens(w: Workload, seed: int, seq: int, tensor: str, t0: int, t1: int,
              factors: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [t1 - t0][Hkv][D] K or V rows of tokens [t0, t1) of sequence seq."""
    if factors is None:
        factors = channel_factors(w, seed, tensor)
    out = []
    c0 = t0 // CHUNK_TOKENS
    c1 = -(-t1 // CHUNK_TOKENS)
    for c in range(c0, c1):
        g = _gen(seed, _name_id(w.name), _TENSOR_ID[tensor], seq, c)
        x = torch.randn(CHUNK_TOKENS, w.kv_heads, w.head_dim, generator=g, dtype=torch.float32)
        lo = max(t0, c * CHUNK_TOKENS) - c * CHUNK_TOKENS
        hi = min(t1, (c + 1) * CHUNK_TOKENS) - c * CHUNK_TOKENS
        out.append((x[lo:hi] * factors).to(torch.bfloat16))
    if not out:
        return torch.empty(0, w.kv_heads, w.head_dim, dtype=torch.bfloat16)
    return torch.cat(out, 0)


def queries(w: Workload, seed: int, step: int = 0) -> torch.Tensor:
    """bf16 [B][Hq][D] query rows, N(0, 1)."""
    g = _gen(seed, _name_id(w.name), _TENSOR_ID["q"], step)
    return torch.randn(w.batch, w.q_heads, w.head_dim, generator=g,
                       dtype=torch.float32).to(torch.bfloat16)


def new_tokens(w: Workload, seed: int, step: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 K and V [B][Hkv][D] of the one token each sequence appends at a
    decode step (paged workload), N(0, 1)."""
    k = kv_tokens(w, seed, 1_000_000 + step, "k", 0, w.batch)
    v = kv_tokens(w, seed, 1_000_000 + step, "v", 0, w.batch)
    return k, v


def seq_lengths(w: Workload, seed: int) -> torch.Tensor:
    """int64 [B] context lengths: fixed for decode/prefill, uniform integers in
    [min_len, max_len] for the paged workload."""
    if w.kind != "paged":
        return torch.full((w.batch,), w.context, dtype=torch.int64)
    g = _gen(seed, _name_id(w.name), _TENSOR_ID["len"])
    return torch.randint(w.min_len, w.max_len + 1, (w.batch,), generator=g, dtype=torch.int64)


@dataclass
class PageTable:
    table: torch.Tensor          # int32 [B][max_pages]; -1 where unused
    num_pages: int               # pages in the pool
    pages_per_seq: List[int]


def identity_page_table(batch: int, tokens_per_seq: int) -> PageTable:
    """Sequence b owns pages b*n .. b*n + n - 1, n = ceil(tokens / 64)."""
    n = -(-tokens_per_seq // PAGE_SIZE)
    t = torch.arange(batch * n, dtype=torch.int32).reshape(batch, n)
    return PageTable(t, batch * n, [n] * batch)


def random_page_table(lengths: torch.Tensor, extra_tokens: int, seed: int, name: str) -> PageTable:
    """Pool = sum of ceil((len_b + extra) / 64) pages, shuffled by a seeded
    permutation and dealt to the sequences in order."""
    need = [-(-(int(l) + extra_tokens) // PAGE_SIZE) for l in lengths.tolist()]
    pool = sum(need)
    g = _gen(seed, _name_id(name), _TENSOR_ID["perm"])
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    maxp = max(need) if need else 1
    t = torch.full((len(need), maxp), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        t[b, :n] = perm[off:off + n]
        off += n
    return PageTable(t, pool, need)


def slots_for(page_table: torch.Tensor, seq: int, t0: int, t1: int) -> torch.Tensor:
    """int64 cache slots (page * 64 + offset) of positions [t0, t1) of a sequence."""
    pos = torch.arange(t0, t1, dtype=torch.int64)
    pages = page_table[seq].to(torch.int64)[pos // PAGE_SIZE]
    return pages * PAGE_SIZE + pos % PAGE_SIZE


def bf16_bits(x: torch.Tensor):
    """uint16 numpy view of a bf16 tensor's bit patterns."""
    import numpy as np
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------- toy sliding-window network

@dataclass(frozen=True)
class ToyNet:
    """A toy multi-layer network of sliding-window attention layers with
    random weights, for the exact-versus-bounded replay study ("Week 6 -- FP4
    KV Caches and Bounded Replay", Overview, Core Concepts and Lab)."""
    name: str
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    batch: int
    tokens: int

    @property
    def d_model(self) -> int:
        return self.q_heads * self.head_dim


TOY_NETS: Dict[str, ToyNet] = {t.name: t for t in [
    ToyNet("toy_swa_l4_w32", layers=4, q_heads=4, kv_heads=2, head_dim=128, window=32, batch=8, tokens=160),
    ToyNet("toy_swa_l1_w32", layers=1, q_heads=4, kv_heads=2, head_dim=128, window=32, batch=4, tokens=80),
    ToyNet("toy_swa_l2_w16", layers=2, q_heads=2, kv_heads=2, head_dim=128, window=16, batch=4, tokens=64),
]}


def toy_weights(t: ToyNet, seed: int):
    """Per layer (W_q [d][Hq*D], W_k [d][Hkv*D], W_v [d][Hkv*D], W_o [Hq*D][d]),
    fp32, N(0, 1/fan_in)."""
    out = []
    d = t.d_model
    for layer in range(t.layers):
        g = _gen(seed, _name_id(t.name), 100 + layer)
        wq = torch.randn(d, t.q_heads * t.head_dim, generator=g) / math.sqrt(d)
        wk = torch.randn(d, t.kv_heads * t.head_dim, generator=g) / math.sqrt(d)
        wv = torch.randn(d, t.kv_heads * t.head_dim, generator=g) / math.sqrt(d)
        wo = torch.randn(t.q_heads * t.head_dim, d, generator=g) / math.sqrt(t.q_heads * t.head_dim)
        out.append((wq, wk, wv, wo))
    return out


def toy_inputs(t: ToyNet, seed: int) -> torch.Tensor:
    """Token embeddings fp32 [B][tokens][d], N(0, 1)."""
    g = _gen(seed, _name_id(t.name), 99)
    return torch.randn(t.batch, t.tokens, t.d_model, generator=g)
