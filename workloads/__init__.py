"""Seeded synthetic inputs for the MoE router / token-dispatch path.

This module only draws random inputs: it holds none of the routing
arithmetic, so both the CPU oracle and the HIP library can be fed from it
without sharing any computation.  Every array is a plain numpy array; bf16
tensors are carried as ``uint16`` arrays holding the bf16 bit patterns.

Recipe (one independent stream per input, so a change to one input never
shifts another):

* ``numpy.random.default_rng([seed, stream])`` with streams
  0 = x, 1 = W, 2 = selection bias, 3 = per-request k, 4 = token ids,
  5 = tid2eid table, 6 = Zipf rank permutation, 7 = expert outputs,
  8 = shared expert output.
* x ~ N(0, 1) and W ~ N(0, 1/d) (std 1/sqrt(d), so logits are ~N(0, 1)),
  drawn as float32; bf16 inputs are the round-to-nearest-even of those
  float32 values.
* Selection bias ~ N(0, variance 0.01), float32.
* Per-request k uniform over {4, 8, 16}, requests of 256 tokens.
* Token ids uniform over the vocabulary; each tid2eid row holds k distinct
  experts drawn uniformly without replacement.
* Skewed load: ``logit_bias[e] = 2.0 * rank_e ** -1.1`` with ranks 1..E
  from a seeded permutation (a Zipf(s=1.1) ranking scaled to 2.0).
* Combine inputs (no trained experts): the expert outputs in dispatch
  order, ``Yp[R][d]``, and a shared expert's output ``[T][d]``, both
  ~N(0, 1) in the workload's dtype -- hidden-state-sized rows, like x.

The routing configurations follow the ones the pages describe: Mixtral
(8 experts, top-2), Qwen3-MoE (128 experts), DeepSeek-V3 (256 experts in
8 groups, keep 4, top-8, sigmoid with a selection bias, scale 2.5),
DeepSeek-V4 (384 experts, top-6, sqrt-softplus, hash routing) and gpt-oss
(128 experts, top-4, softmax over the selected logits).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

(STREAM_X, STREAM_W, STREAM_BIAS, STREAM_K, STREAM_TOK, STREAM_TABLE, STREAM_ZIPF,
 STREAM_YP, STREAM_SHARED) = range(9)

# score-function names shared by both sides as plain strings
SCORES = ("softmax", "sigmoid", "sqrt_softplus", "softmax_topk")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int                      # fixed k, or k_max when k varies per request
    dtype: str                  # "f32" or "bf16" (x and W)
    score: str
    n_groups: int = 1
    topk_groups: int = 1
    group_score: str = "max"    # "max" or "top2_sum"
    renormalize: bool = True
    route_scale: float = 1.0
    select_bias: bool = False   # draw a selection-only bias ~N(0, 0.01)
    dynamic_k: tuple = ()       # per-request k choices; empty = fixed k
    request_len: int = 256
    zipf_offsets: bool = False  # add Zipf logit offsets (skewed load)
    zipf_s: float = 1.1
    zipf_scale: float = 2.0
    hash_vocab: int = 0         # >0: hash routing over this vocabulary
    capacity_factor: float = 0  # >0: capacity-limited dispatch, C = ceil(f * T * k / E)
    k_per_group: int = 0        # >0: grouped top-k, at most this many per group

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=int(T))


WORKLOADS = {
    # Mixtral-like: 8 experts, top-2, softmax over all logits then renorm.
    "mixtral": Workload("mixtral", T=256, d=1024, E=8, k=2, dtype="f32",
                        score="softmax"),
    # Qwen3-MoE-like with a per-request k in {4, 8, 16}: 16 requests of 256.
    "qwen3_dynk": Workload("qwen3_dynk", T=4096, d=2048, E=128, k=16,
                           dtype="bf16", score="softmax", dynamic_k=(4, 8, 16)),
    # DeepSeek-V3-like: sigmoid, selection bias, 8 groups keep 4, top-8, x2.5.
    "dsv3_grouped": Workload("dsv3_grouped", T=8192, d=7168, E=256, k=8,
                             dtype="bf16", score="sigmoid", n_groups=8,
                             topk_groups=4, group_score="top2_sum",
                             route_scale=2.5, select_bias=True),
    # DeepSeek-V4-like: 384 experts, top-6, sqrt(softplus) renormalised.
    "dsv4": Workload("dsv4", T=16384, d=7168, E=384, k=6, dtype="bf16",
                     score="sqrt_softplus"),
    # DeepSeek-V4-like hash layer: ids from a [129280][6] token->expert table.
    "dsv4_hash": Workload("dsv4_hash", T=16384, d=7168, E=384, k=6,
                          dtype="bf16", score="sqrt_softplus",
                          hash_vocab=129280),
    # gpt-oss-like large prefill, skewed by Zipf logit offsets.
    "gptoss_skew": Workload("gptoss_skew", T=65536, d=2880, E=128, k=4,
                            dtype="bf16", score="softmax_topk",
                            zipf_offsets=True),
    # Routing variants on the same kernels.  DeepSeek-V4-like with the
    # selection-only bias and a weight scale (sqrt-softplus + bias, weights
    # from the unbiased scores, renormalised, then scaled; the scale's value
    # is not given, 1.5 stands in).
    "dsv4_bias": Workload("dsv4_bias", T=16384, d=7168, E=384, k=6, dtype="bf16",
                          score="sqrt_softplus", select_bias=True, route_scale=1.5),
    # OLMoE-like: softmax over all 64 experts, top-8, probabilities kept as
    # they are (not renormalised).
    "olmoe": Workload("olmoe", T=4096, d=2048, E=64, k=8, dtype="bf16", score="softmax",
                      renormalize=False),
    # DeepSeek-V3-like grouping without a bias: each group scored by its
    # largest sigmoid, keep 4 of 8, top-8, renormalised x2.5.
    "dsv3_groupmax": Workload("dsv3_groupmax", T=8192, d=7168, E=256, k=8, dtype="bf16",
                              score="sigmoid", n_groups=8, topk_groups=4, group_score="max",
                              route_scale=2.5),
    # Top-1 of 128 routed experts (Llama-4-Maverick-like) with an expert
    # capacity in the manner of the Switch Transformer: the chosen expert's
    # softmax probability as its weight, capacity ceil(1.25 * T * k / E); the
    # hidden size is not given, 4096 stands in.
    "switch_top1": Workload("switch_top1", T=16384, d=4096, E=128, k=1, dtype="bf16",
                            score="softmax", renormalize=False, capacity_factor=1.25),
    # Grouped top-k with a per-group quota (ferrox_moe route_top_k_grouped):
    # the DeepSeek-V3-like shape and 8 groups, the 2 best of each group, then
    # the global top-8 of those 16, sigmoid scores renormalised.  The page
    # gives no sizes; these stand in.
    "grouped_quota": Workload("grouped_quota", T=8192, d=7168, E=256, k=8, dtype="bf16",
                              score="sigmoid", n_groups=8, topk_groups=8, k_per_group=2),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def normal_f32(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    a = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def draw_matrix(seed: int, stream: int, shape, std: float, dtype: str) -> np.ndarray:
    a = normal_f32(seed, stream, shape, std)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def zipf_offsets(seed: int, E: int, s: float = 1.1, scale: float = 2.0) -> np.ndarray:
    """Per-expert logit offsets ``scale * rank^-s``, ranks 1..E in seeded order."""
    ranks = rng(seed, STREAM_ZIPF).permutation(E).astype(np.float64) + 1.0
    return (scale * ranks ** (-s)).astype(np.float32)


def request_k(seed: int, T: int, choices, request_len: int = 256) -> np.ndarray:
    """Per-token k from per-request draws: token t belongs to request t // request_len."""
    n_req = (T + request_len - 1) // request_len
    kr = rng(seed, STREAM_K).choice(np.asarray(choices, dtype=np.int32), size=n_req)
    return np.repeat(kr, request_len)[:T].astype(np.int32)


def token_ids(seed: int, T: int, vocab: int) -> np.ndarray:
    return rng(seed, STREAM_TOK).integers(0, vocab, size=T, dtype=np.int64).astype(np.int32)


def tid2eid_table(seed: int, vocab: int, k: int, E: int) -> np.ndarray:
    """[vocab][k] int32, each row k distinct experts uniform without replacement.

    Rows with a repeated expert are redrawn (rejection), which keeps every
    row uniform over the k-subsets in a uniformly random order."""
    if k > E:
        raise ValueError("k distinct experts need k <= E")
    g = rng(seed, STREAM_TABLE)
    tab = g.integers(0, E, size=(vocab, k), dtype=np.int64)

    def dup_rows(t):
        s = np.sort(t, axis=1)
        return np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0]

    bad = dup_rows(tab)
    while bad.size:
        tab[bad] = g.integers(0, E, size=(bad.size, k), dtype=np.int64)
        bad = bad[np.asarray(dup_rows(tab[bad]), dtype=np.int64)]
    return tab.astype(np.int32)


def make_inputs(w: Workload, seed: int = 0, T: Optional[int] = None) -> dict:
    """All inputs of one workload as numpy arrays (x, W, biases, k, tokens, table)."""
    if T is not None:
        w = w.with_T(T)
    out = {"workload": w, "seed": seed}
    out["x"] = draw_matrix(seed, STREAM_X, (w.T, w.d), 1.0, w.dtype)
    out["W"] = draw_matrix(seed, STREAM_W, (w.E, w.d), 1.0 / np.sqrt(w.d), w.dtype)
    out["select_bias"] = (normal_f32(seed, STREAM_BIAS, (w.E,), 0.1)
                          if w.select_bias else None)
    out["logit_bias"] = (zipf_offsets(seed, w.E, w.zipf_s, w.zipf_scale)
                         if w.zipf_offsets else None)
    out["k_per_token"] = (request_k(seed, w.T, w.dynamic_k, w.request_len)
                          if w.dynamic_k else None)
    if w.hash_vocab:
        out["token_ids"] = token_ids(seed, w.T, w.hash_vocab)
        out["tid2eid"] = tid2eid_table(seed, w.hash_vocab, w.k, w.E)
    return out


def capacity(w: Workload) -> int:
    """Expert capacity of a capacity-limited workload: ceil(f * T * k / E)."""
    return int(np.ceil(w.capacity_factor * w.T * w.k / w.E))


def expert_outputs(w: Workload, R: int, seed: int = 0) -> np.ndarray:
    """Yp[R][d]: synthetic expert outputs in dispatch order (workload dtype)."""
    return draw_matrix(seed, STREAM_YP, (int(R), w.d), 1.0, w.dtype)


def shared_output(w: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """[T][d]: a synthetic shared expert's output (workload dtype)."""
    return draw_matrix(seed, STREAM_SHARED, (w.T if T is None else int(T), w.d), 1.0, w.dtype)


def rows(x: np.ndarray, idx) -> np.ndarray:
    """Gather rows (a sample of tokens) keeping the array's dtype."""
    return np.ascontiguousarray(x[np.asarray(idx)])
