"""Seeded synthetic inputs for MoE expert-parallel dispatch/combine.

This module only draws inputs: routing ids, routing weights, token rows and
the stand-in expert parameters. It holds none of the dispatch/combine
arithmetic and is shared by the tests, the benchmark and the oracle's
callers so that both sides see byte-identical inputs.

Shapes follow the MoE workloads of "Enabling trillion-parameter models on
AWS EFA" (section "Evaluation", dispatch/combine latency): hidden size 7168,
block-scaled fp8 dispatch, bf16 combine, decode batch 128 and prefill batch
4096 tokens per rank. N ranks each hold T tokens; each token picks R of E
experts, and expert e lives on rank e // (E // N).

Draw order for every workload (one numpy Generator per workload):
routing ids, then weight logits, then token values, then expert scales.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

PAYLOAD_BF16 = 0
PAYLOAD_FP8_B128 = 1
FP8_BLOCK = 128
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Shape:
    """Problem shape plus the routing/expert recipe of one workload."""

    name: str
    n_ranks: int        # N
    tokens: int         # T, tokens per rank
    hidden: int         # H
    n_experts: int      # E
    topk: int           # R
    routing: str = "uniform"     # uniform | zipf | rank0 | custom
    payload: int = PAYLOAD_BF16  # PAYLOAD_BF16 | PAYLOAD_FP8_B128
    expert: str = "identity"     # identity | scale | dequant
    seed: int = 0
    zipf_s: float = 1.2
    cap_rows: int = 0            # 0 means the worst-case receive bound

    @property
    def local_experts(self) -> int:
        return self.n_experts // self.n_ranks


# The five workloads. The first is small enough for an exhaustive CPU check;
# the second (decode scale) is the one the benchmark times.
CONFIGS = {
    "tiny": Shape("tiny", 4, 16, 256, 16, 2),
    "decode": Shape("decode", 32, 128, 7168, 256, 8, expert="scale"),
    "tiny_zipf": Shape("tiny_zipf", 4, 16, 256, 16, 2, routing="zipf"),
    "prefill": Shape("prefill", 8, 4096, 7168, 256, 8,
                     payload=PAYLOAD_FP8_B128, expert="dequant"),
    "worst": Shape("worst", 64, 128, 7168, 384, 8, routing="rank0"),
    # The Zipf recipe also at decode shapes: the skewed-routing workload read
    # as "decode shapes" rather than "tiny shapes".
    "decode_zipf": Shape("decode_zipf", 32, 128, 7168, 256, 8,
                         routing="zipf", expert="scale"),
    # Decode shapes with the block-scaled fp8 dispatch of the evaluation
    # setting (quantised by the sender, dequantised by the stand-in expert).
    "decode_fp8": Shape("decode_fp8", 32, 128, 7168, 256, 8,
                        payload=PAYLOAD_FP8_B128, expert="dequant"),
}


@dataclasses.dataclass
class Workload:
    shape: Shape
    idx: np.ndarray                 # int32 [N, T, R]
    weights: np.ndarray             # float32 [N, T, R]
    x_bf16: np.ndarray              # uint16 [N, T, H], bf16 bit patterns
    planes: list                    # dispatch payload planes, uint8 [N, T, row_p]
    alpha: Optional[np.ndarray]     # float32 [E] for the "scale" expert


def _draw_routing(rng: np.random.Generator, sh: Shape) -> np.ndarray:
    N, T, E, R = sh.n_ranks, sh.tokens, sh.n_experts, sh.topk
    if sh.routing == "uniform":
        # R distinct experts per token, uniformly, in random order: the first
        # R entries of a uniformly random permutation of the E experts.
        keys = rng.random((N, T, E))
        return np.argsort(keys, axis=-1, kind="stable")[..., :R].astype(np.int32)
    if sh.routing == "zipf":
        # Zipf popularity over a seeded expert permutation, then R distinct
        # experts per token by successive weighted sampling without
        # replacement (Gumbel-top-k: the key order is the draw order).
        perm = rng.permutation(E)
        p = np.empty(E)
        p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-sh.zipf_s)
        p /= p.sum()
        keys = np.log(p)[None, None, :] + rng.gumbel(size=(N, T, E))
        return np.argsort(-keys, axis=-1, kind="stable")[..., :R].astype(np.int32)
    if sh.routing == "rank0":
        # Every slot goes to an expert hosted on rank 0. With R > E/N the
        # ids of one token repeat: the first min(R, L) slots are a random
        # permutation of rank 0's experts, the rest distinct draws again.
        L = sh.local_experts
        if L <= 0:
            raise ValueError("rank0 routing needs E >= N")
        cols = []
        left = R
        while left > 0:
            take = min(left, L)
            keys = rng.random((N, T, L))
            cols.append(np.argsort(keys, axis=-1, kind="stable")[..., :take])
            left -= take
        return np.concatenate(cols, axis=-1).astype(np.int32)
    raise ValueError(f"unknown routing {sh.routing!r}")


def _draw_weights(rng: np.random.Generator, sh: Shape) -> np.ndarray:
    logits = rng.standard_normal((sh.n_ranks, sh.tokens, sh.topk))
    z = np.exp(logits - logits.max(axis=-1, keepdims=True))
    return (z / z.sum(axis=-1, keepdims=True)).astype(np.float32)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_fp8_b128(x_bf16: np.ndarray):
    """Block-scaled fp8 input preparation (not part of the library).

    One fp32 scale per 128 consecutive elements of a row: scale = amax / 448
    (1 for an all-zero block); codes are OCP e4m3fn of x / scale, rounded to
    nearest even and clamped to +-448. Returns (codes uint8 [..., H],
    scales float32 [..., H/128]).
    """
    x = bf16_bits_to_f32(x_bf16)
    shp = x.shape
    H = shp[-1]
    assert H % FP8_BLOCK == 0
    xb = x.reshape(*shp[:-1], H // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(xb).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    q = np.clip(xb / scale[..., None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn)
    codes = codes.view(torch.uint8).numpy().reshape(shp)
    return codes, scale


def make_workload(sh: Shape, idx: Optional[np.ndarray] = None) -> Workload:
    """Draw one workload. `idx` overrides the routing (for edge cases)."""
    rng = np.random.default_rng(sh.seed)
    N, T, H = sh.n_ranks, sh.tokens, sh.hidden
    if idx is None:
        idx = _draw_routing(rng, sh)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.shape == (N, T, sh.topk)
    weights = _draw_weights(rng, sh)
    x = rng.standard_normal((N, T, H), dtype=np.float32)
    x_bf16 = to_bf16_bits(x)
    del x
    alpha = None
    if sh.expert == "scale":
        alpha = rng.uniform(0.5, 1.5, size=sh.n_experts).astype(np.float32)
    if sh.payload == PAYLOAD_BF16:
        planes = [x_bf16.view(np.uint8).reshape(N, T, 2 * H)]
    elif sh.payload == PAYLOAD_FP8_B128:
        codes, scales = quantize_fp8_b128(x_bf16)
        planes = [codes.reshape(N, T, H),
                  scales.view(np.uint8).reshape(N, T, 4 * (H // FP8_BLOCK))]
    else:
        raise ValueError(sh.payload)
    return Workload(sh, idx, weights, x_bf16, planes, alpha)


# ---------------------------------------------------------------------------
# KV-block push workloads (the prefill-to-decode KV transfer)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class KvShape:
    """One request's KV moved to `ranks` tensor-parallel ranks. Each side
    keeps a pool of `*_pool_blocks` blocks of `*_block_tokens` tokens of
    `token_bytes` bytes (all layers of a token together); its free list is
    fragmented into runs of consecutive blocks with the given mean length."""
    name: str
    ranks: int
    tokens: int
    token_bytes: int
    src_block_tokens: int
    dst_block_tokens: int
    src_pool_blocks: int
    dst_pool_blocks: int
    src_mean_run: float = 256.0
    dst_mean_run: float = 32.0
    seed: int = 0


KV_CONFIGS = {
    "kv_tiny": KvShape("kv_tiny", 2, 37, 64, 4, 1, 40, 120, 3.0, 2.0),
    # The push-connector page's setting: Qwen3-32B served with tensor
    # parallelism 8 (64 layers, 8 KV heads of 128, bf16: one KV head per
    # rank, K and V, 64 x 2 x 128 x 2 B = 32 KiB per token per rank), a
    # 16k-token prompt (the longest of its 1k-16k sweep), vLLM's 16-token
    # blocks; free lists fragmented into runs of 64 (prefill) and 8 (decode)
    # blocks on average.
    "kv_qwen32b_16k": KvShape("kv_qwen32b_16k", 8, 16384, 32768, 16, 16, 2048, 2048, 64.0, 8.0),
    # The same request size with page size 1 (the SGLang setting of the
    # shm / SAR page), 4096 tokens.
    "kv_page1_4k": KvShape("kv_page1_4k", 8, 4096, 32768, 1, 1, 16384, 16384, 256.0, 32.0),
}


def _free_list(rng: np.random.Generator, blocks: int, mean_run: float) -> np.ndarray:
    """Pool block ids cut into runs of consecutive ids (geometric lengths of
    the given mean), runs in random order."""
    cuts, pos = [], 0
    while pos < blocks:
        n = int(rng.geometric(1.0 / max(mean_run, 1.0)))
        cuts.append((pos, min(blocks, pos + n)))
        pos += n
    order = rng.permutation(len(cuts))
    return np.concatenate([np.arange(*cuts[i]) for i in order]).astype(np.int32)


def make_kv_tables(sh: KvShape):
    """Block tables (source, destination) of the request."""
    rng = np.random.default_rng(sh.seed)
    ns = -(-sh.tokens // sh.src_block_tokens)
    nd = -(-sh.tokens // sh.dst_block_tokens)
    src = _free_list(rng, sh.src_pool_blocks, sh.src_mean_run)[:ns]
    dst = _free_list(rng, sh.dst_pool_blocks, sh.dst_mean_run)[:nd]
    assert len(src) == ns and len(dst) == nd, "pool too small for the request"
    return src, dst
