"""Seeded synthetic inputs for the AFD FFN-rank hot path.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic.  Both the HIP path (through the tests and the
benchmark) and the CPU oracle consume what it returns, and neither side
generates inputs of its own.

Workloads (named by shape; P peers with seq_lens, T = sum(seq_lens)):

  tiny      P=2 [7,13]                    H=64   E=8   K=2 I=32   Is=32
  prefill   P=2 [1024,3072]               H=2048 E=64  K=6 I=1408 Is=2816
  fanin4    P=4 [3296,2682,4976,3242]     H=2048 E=64  K=6 I=1408 Is=2816
  skew      P=2 [4096,4096]               H=7168 E=256 K=8 I=2048 Is=2048
  decode    P=8 [16]*8                    H=2048 E=64  K=6 I=1408 Is=2816

The fanin4 lengths are the seed-0 draw of lognormal(mu=8, sigma=0.8) for four
peers, rounded to integers and clipped to [64, 8192].  The skew workload adds a
per-expert bias of -1.1*ln(e+1) (the log of a Zipf(s=1.1) popularity with rank
e+1) to the router logits, so expert load is imbalanced.

Two recipes, both seeded (seed 0 by default):

  "stream"  one numpy PCG64 stream default_rng(seed) drawing, in order,
            X ~ N(0,1) [T,H], L ~ N(0,1) [T,E], W13 = 0.02*N [E,2I,H],
            W2 = 0.02*N [E,H,I], Ws13 = 0.02*N [2Is,H], Ws2 = 0.02*N [H,Is],
            all float32, then rounded to bf16 (round to nearest even).
  "chunked" the same distributions, but each tensor (and each expert's slice
            of W13 / W2) draws from its own child stream
            default_rng([seed, tensor_id, expert]) so that the draw can run on
            many threads; used for the large workloads, where one stream would
            take minutes on one core.

Hidden states and weights are returned as bf16 bit patterns (uint16); logits
as float32.  Weight layouts: W13 [E][2I][H] (rows [0,I) gate, [I,2I) up),
W2 [E][H][I], Ws13 [2Is][H], Ws2 [H][Is].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seq_lens: tuple
    hidden: int
    num_experts: int
    top_k: int
    intermediate: int
    shared_intermediate: int
    token_cap: int
    zipf_bias: float = 0.0          # s of the Zipf per-expert logit bias (0 = none)
    routed_scaling_factor: float = 1.0
    renormalize: int = 1
    recipe: str = "chunked"
    seed: int = 0
    ring_depth: int = 1
    attention_routes: int = 0       # 1: the attention side routes (grouped routed rows, sender combines)
    route_experts: int = 0          # experts the peers route over when the window owns a segment (0: all)
    expert_offset: int = 0          # first expert of the window's segment
    w1_fp8: int = 0                 # 1: gate/up GEMMs on e4m3 operands
    notes: str = field(default="", compare=False)

    @property
    def num_peers(self) -> int:
        return len(self.seq_lens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


FANIN4_SEQ_LENS = (3296, 2682, 4976, 3242)

WORKLOADS = {
    "tiny": Workload("tiny", (7, 13), 64, 8, 2, 32, 32, token_cap=16, recipe="stream"),
    "prefill": Workload("prefill", (1024, 3072), 2048, 64, 6, 1408, 2816, token_cap=4096),
    "fanin4": Workload("fanin4", FANIN4_SEQ_LENS, 2048, 64, 6, 1408, 2816, token_cap=8192),
    "skew": Workload("skew", (4096, 4096), 7168, 256, 8, 2048, 2048, token_cap=4096,
                     zipf_bias=1.1),
    "decode": Workload("decode", (16,) * 8, 2048, 64, 6, 1408, 2816, token_cap=16),
}


def fanin4_seq_lens(seed: int = 0) -> tuple:
    """The fanin4 peer lengths: lognormal(8, 0.8) x 4, rounded, clipped."""
    r = np.random.default_rng(seed).lognormal(8.0, 0.8, 4)
    return tuple(int(v) for v in np.clip(np.rint(r), 64, 8192))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def _normal_bf16(rng, shape, scale) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return bf16_bits(a)


def _chunked_experts(seed, tid, E, shape, scale, pool) -> np.ndarray:
    out = np.empty((E,) + shape, dtype=np.uint16)

    def one(e):
        out[e] = _normal_bf16(np.random.default_rng([seed, tid, e]), shape, scale)

    list(pool.map(one, range(E)))
    return out


def make_inputs(wl: Workload, with_weights: bool = True, progress=None) -> dict:
    """Draw the inputs of one workload.

    Returns a dict with X (uint16 [T,H]), L (float32 [T,E]), the per-peer
    views x[p] / l[p], and (with_weights) W13, W2, Ws13, Ws2 as uint16.
    """
    T, H, E, I, Is = wl.total_tokens, wl.hidden, wl.num_experts, wl.intermediate, wl.shared_intermediate
    out = {"workload": wl, "seq_lens": np.asarray(wl.seq_lens, dtype=np.int32)}
    if wl.recipe == "stream":
        rng = np.random.default_rng(wl.seed)
        X = _normal_bf16(rng, (T, H), 1.0)
        L = rng.standard_normal((T, E), dtype=np.float32)
        if with_weights:
            out["W13"] = _normal_bf16(rng, (E, 2 * I, H), 0.02)
            out["W2"] = _normal_bf16(rng, (E, H, I), 0.02)
            if Is > 0:
                out["Ws13"] = _normal_bf16(rng, (2 * Is, H), 0.02)
                out["Ws2"] = _normal_bf16(rng, (H, Is), 0.02)
    elif wl.recipe == "chunked":
        X = _normal_bf16(np.random.default_rng([wl.seed, 0]), (T, H), 1.0)
        L = np.random.default_rng([wl.seed, 1]).standard_normal((T, E), dtype=np.float32)
        if with_weights:
            with ThreadPoolExecutor(_threads()) as pool:
                if progress:
                    progress("W13")
                out["W13"] = _chunked_experts(wl.seed, 2, E, (2 * I, H), 0.02, pool)
                if progress:
                    progress("W2")
                out["W2"] = _chunked_experts(wl.seed, 3, E, (H, I), 0.02, pool)
            if Is > 0:
                out["Ws13"] = _normal_bf16(np.random.default_rng([wl.seed, 4]), (2 * Is, H), 0.02)
                out["Ws2"] = _normal_bf16(np.random.default_rng([wl.seed, 5]), (H, Is), 0.02)
    else:
        raise ValueError(f"unknown recipe {wl.recipe!r}")
    if wl.zipf_bias:
        bias = (-wl.zipf_bias * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        L = L + bias[None, :]
    out["X"], out["L"] = X, np.ascontiguousarray(L, dtype=np.float32)
    off = np.concatenate([[0], np.cumsum(wl.seq_lens)]).astype(np.int64)
    out["x"] = [X[off[p]:off[p + 1]] for p in range(wl.num_peers)]
    out["l"] = [out["L"][off[p]:off[p + 1]] for p in range(wl.num_peers)]
    return out


def small_workload(name="ragged", seq_lens=(37, 0, 211, 96), hidden=256, num_experts=12,
                   top_k=3, intermediate=200, shared_intermediate=136, token_cap=256,
                   **kw) -> Workload:
    """A workload the oracle finishes in seconds that still spans several GEMM
    tiles with ragged tails (default: an empty peer, non-multiple-of-64 widths)."""
    return Workload(name, tuple(seq_lens), hidden, num_experts, top_k, intermediate,
                    shared_intermediate, token_cap=token_cap, recipe="chunked", **kw)
