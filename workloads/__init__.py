"""Seeded synthetic inputs for MoE dispatch / combine.

This module only draws random inputs; it holds none of the method's
arithmetic (no counts, prefix sums, ranks, copies, quantisation or weighted
sums) and imports neither the oracle nor the HIP library, so both sides of a
parity test can take their inputs from it.

Workloads follow the shapes the pages describe: hidden size 7168 (the Ascend
A3 combine constraint on H), top-8 routing (its K limit) over 256 or 512 experts
(its expert-count range), decode-sized and prefill-sized batches, skewed
expert popularity (the DeepEP PR tests a skew of 0.6) and a mixed regime with a
few hot experts above 1000 tokens and many cold ones under the ~160-token
flat-regime threshold (TEMPO summary, section 1).  No routing trace or trained
weights are used: everything is drawn from seeded generators.

Recipe (fixed, so results reproduce across machines):

* Seeds: ``numpy.random.SeedSequence(seed).spawn(5)`` gives the child streams
  routing, logits, x, y, shared, in that order.
* Uniform routing: per token, the K largest of E i.i.d. U(0,1) keys, in
  descending key order (a uniformly random ordered K-subset).
* Zipf(alpha) routing without replacement: expert ``perm[i]`` has popularity
  proportional to ``(i+1)**-alpha`` over a seeded permutation ``perm``; per
  token the top K of ``log p + Gumbel(0,1)`` keys, descending (equivalent to
  sequential sampling without replacement).
* Scales: softmax (computed in float64, stored float32) of K i.i.d. N(0,1)
  logits per token -- the full softmax renormalised over the chosen K.
* Rows (x, y, shared): N(0,1) float32 from a seeded torch CPU generator,
  rounded to bfloat16 by torch, drawn in fixed row chunks.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

CHUNK_ELEMS = 1 << 25  # rows are drawn in chunks of about this many elements


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    bs: int
    hidden: int
    experts: int
    topk: int
    routing: str            # "uniform" | "zipf"
    alpha: float = 0.0      # Zipf exponent
    fp8: bool = False       # dispatch quantises to e4m3
    identity_experts: bool = False  # y is the dispatched buffer itself
    shared: bool = True     # a shared-expert row is added
    seed: int = 0
    align: int = 128


WORKLOADS = {
    "tiny": Workload("tiny", bs=16, hidden=128, experts=8, topk=2, routing="uniform",
                     identity_experts=True, shared=False, seed=0),
    "decode": Workload("decode", bs=128, hidden=7168, experts=256, topk=8, routing="uniform",
                       seed=1),
    "skewed": Workload("skewed", bs=4096, hidden=7168, experts=256, topk=8, routing="zipf",
                       alpha=0.6, seed=2),
    "fp8": Workload("fp8", bs=4096, hidden=7168, experts=256, topk=8, routing="uniform",
                    fp8=True, seed=3),
    "large": Workload("large", bs=16384, hidden=7168, experts=512, topk=8, routing="zipf",
                      alpha=1.2, seed=4),
}

_STREAMS = ("routing", "logits", "x", "y", "shared")


def seed_streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, children))


def _torch_seed(ss: np.random.SeedSequence) -> int:
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def routing(bs: int, experts: int, topk: int, kind: str = "uniform", alpha: float = 0.0,
            seed: int = 0) -> np.ndarray:
    """int32 [bs, topk] expert ids, distinct within each row."""
    rng = np.random.default_rng(seed_streams(seed)["routing"])
    if kind == "uniform":
        keys = rng.random((bs, experts))
    elif kind == "zipf":
        perm = rng.permutation(experts)
        logp = np.empty(experts)
        logp[perm] = -alpha * np.log(np.arange(1, experts + 1, dtype=np.float64))
        keys = logp[None, :] + rng.gumbel(size=(bs, experts))
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    order = np.argsort(-keys, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :topk], dtype=np.int32)


def scales(bs: int, topk: int, seed: int = 0) -> np.ndarray:
    """float32 [bs, topk]: softmax of N(0,1) logits over the chosen K."""
    rng = np.random.default_rng(seed_streams(seed)["logits"])
    logits = rng.standard_normal((bs, topk))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def bf16_rows(rows: int, cols: int, seed: int, stream: str = "x") -> torch.Tensor:
    """bfloat16 [rows, cols] CPU tensor of N(0,1) values."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(_torch_seed(seed_streams(seed)[stream]))
    out = torch.empty((rows, cols), dtype=torch.bfloat16)
    step = max(1, CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = torch.randn((r1 - r0, cols), generator=gen, dtype=torch.float32).to(
            torch.bfloat16)
    return out


def e4m3_rows(rows: int, cols: int, seed: int, stream: str = "y"):
    """Expert-output rows in e4m3 form: uint8 codes [rows, cols] and fp32
    scales [rows, cols/128].  Codes are N(0,1)*64 values cast to float8_e4m3fn
    by torch (saturating to +-448); scales are U(1e-3, 2e-2).  The values are
    only realistic-looking inputs; no quantisation rule of the method is used."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(_torch_seed(seed_streams(seed)[stream]) ^ 0x5DEECE66D)
    codes = torch.empty((rows, cols), dtype=torch.uint8)
    step = max(1, CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        v = torch.randn((r1 - r0, cols), generator=gen, dtype=torch.float32) * 64.0
        codes[r0:r1] = v.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = torch.rand((rows, cols // 128), generator=gen, dtype=torch.float32) * 0.019 + 0.001
    return codes, scales


def popularity(experts: int, kind: str = "zipf", seed: int = 0) -> np.ndarray:
    """Experts from most to least popular under the workload's Zipf draw (the
    same seeded permutation ``routing`` uses); uniform routing has no order."""
    if kind != "zipf":
        return np.arange(experts)
    rng = np.random.default_rng(seed_streams(seed)["routing"])
    return rng.permutation(experts)


def replica_plan(experts: int, hot: np.ndarray, replicas_per_hot: int):
    """A synthetic replica table: each expert in ``hot`` gets
    ``replicas_per_hot`` physical replicas chosen with equal probability, every
    other expert one.  Returns (offsets int32 [E+1], thresholds uint32 [P]) in
    the cumulative-threshold form the replica-aware layout takes."""
    reps = np.ones(experts, np.int64)
    reps[np.asarray(hot, np.int64)] = replicas_per_hot
    offsets = np.concatenate([[0], np.cumsum(reps)]).astype(np.int32)
    thresholds = np.empty(int(offsets[-1]), np.uint32)
    for e in range(experts):
        g = int(reps[e])
        cuts = [((j + 1) * (1 << 32)) // g - 1 for j in range(g)]
        thresholds[offsets[e]:offsets[e + 1]] = np.array(cuts, np.uint64).astype(np.uint32)
    return offsets, thresholds


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a CPU bfloat16 tensor (a view, no copy)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def make(w: Workload | str, *, rows_y: int | None = None, seed: int | None = None,
         with_rows: bool = True) -> dict:
    """All inputs of one workload as CPU arrays/tensors.

    ``rows_y`` is the number of expert-output rows to draw (the caller sizes it
    from the library's or the oracle's capacity rule); ``None`` skips y.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    s = w.seed if seed is None else seed
    out = {
        "workload": w,
        "expert_ids": routing(w.bs, w.experts, w.topk, w.routing, w.alpha, s),
        "expert_scales": scales(w.bs, w.topk, s),
    }
    if with_rows:
        out["x"] = bf16_rows(w.bs, w.hidden, s, "x")
        out["shared"] = bf16_rows(w.bs, w.hidden, s, "shared") if w.shared else None
        if rows_y is not None and not w.identity_experts:
            out["y"] = bf16_rows(rows_y, w.hidden, s, "y")
    return out
