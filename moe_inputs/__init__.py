"""Seeded synthetic workloads for the token-choice MoE FFN layer forward pass.

This module only draws random numbers and lays them out. It holds none of the
layer's arithmetic (no routing, no capacity, no FFN, no output rounding), so
both the CPU oracle and the HIP path can read the same arrays without sharing
any of the method's code.

Shapes follow the models the pages name: Mixtral 8x7B (8 experts, top-2,
SwiGLU) in "How do Mixture of Expert Models Work?" section "The Math Behind
MoEs"; OpenMoE-8B (32 experts, 2 active) in the OpenMoE issue page; 64 experts
choose 8 ("fine-grained") in the same issue page. The skewed workload emulates
the "Context-independent Specialization" finding in "Take a Closer Look at the
MoE LLM Routing" (Introduction): tokens that share a token id go to the same
few experts.

Streams: numpy.random.SeedSequence(seed).spawn(E + 2) gives independent
PCG64 streams, so experts can be drawn in parallel threads and the result
does not depend on the thread count:
  stream 0      router weight W_g, drawn as (d, E) / sqrt(d)
  stream 1 + e  expert e: W_gate_e (d, F) / sqrt(d), then W_up_e (d, F) / sqrt(d),
                then W_down_e (F, d) / sqrt(d)
  stream E + 1  the token-side draws (x, or ids / per-id vectors / noise for
                "zipf").
Each matrix is then transposed into the library layout [out, in] (the input
dimension contiguous) and, for bf16 workloads, rounded to bfloat16 with
torch's own conversion (a library routine, round-to-nearest-even).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens in the routing group
    d: int            # hidden size
    E: int            # experts
    k: int            # experts per token
    F: int            # expert FFN width (SwiGLU)
    cf: float         # capacity factor; 0.0 means dropless
    dtype: str        # "f32" or "bf16": storage type of x, weights, h, o, y
    seed: int
    gen: str = "normal"   # "normal" or "zipf"
    zipf_s: float = 1.1
    zipf_vocab: int = 32768
    zipf_alpha: float = 1.0
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=64, d=64, E=4, k=1, F=128, cf=1.25,
                          dtype="f32", seed=0,
                          note="tiny fp32 layer, capacity factor 1.25"),
    "mixtral_bf16": Workload("mixtral_bf16", T=4096, d=4096, E=8, k=2, F=14336,
                             cf=0.0, dtype="bf16", seed=1,
                             note="Mixtral-shaped layer, dropless"),
    "openmoe_bf16": Workload("openmoe_bf16", T=8192, d=2048, E=32, k=2, F=8192,
                             cf=1.25, dtype="bf16", seed=2, gen="zipf",
                             note="OpenMoE-shaped layer, Zipf(1.1) token ids, cf 1.25"),
    "finegrained_bf16": Workload("finegrained_bf16", T=8192, d=2048, E=64, k=8,
                                 F=1408, cf=0.0, dtype="bf16", seed=3,
                                 note="64 experts choose 8, dropless"),
    "decode_bf16": Workload("decode_bf16", T=32, d=4096, E=8, k=2, F=14336,
                            cf=0.0, dtype="bf16", seed=1,
                            note="decode batch of 32 on the Mixtral-shaped weights"),
}


def _storage(a32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def _storage_t(a32: np.ndarray, dtype: str) -> torch.Tensor:
    """Transpose a drawn (in, out) matrix into the [out, in] layout, then store."""
    t = torch.from_numpy(a32)
    if dtype == "bf16":
        return t.to(torch.bfloat16).T.contiguous()
    if dtype == "f32":
        return t.T.contiguous()
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, scale: float | None = None) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale is not None:
        a *= np.float32(scale)
    return a


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload, expert_weights: bool = True) -> dict:
    """Draw one workload. Returns CPU torch tensors in the storage dtype:

    x        [T, d]
    w_router [E, d]
    w_gate   [E, F, d]   (None when expert_weights=False)
    w_up     [E, F, d]
    w_down   [E, d, F]
    token_ids [T]        ("zipf" workloads only)
    """
    ss = np.random.SeedSequence(w.seed).spawn(w.E + 2)
    inv = 1.0 / math.sqrt(w.d)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    wr = _normal(np.random.default_rng(ss[0]), (w.d, w.E), inv)
    out = {"w_router": _storage(wr.T, w.dtype)}
    if expert_weights:
        wg = torch.empty((w.E, w.F, w.d), dtype=tdt)
        wu = torch.empty((w.E, w.F, w.d), dtype=tdt)
        wd = torch.empty((w.E, w.d, w.F), dtype=tdt)

        def one(e):
            rng = np.random.default_rng(ss[1 + e])
            g = _normal(rng, (w.d, w.F), inv)
            wg[e].copy_(_storage_t(g, w.dtype))
            del g
            u = _normal(rng, (w.d, w.F), inv)
            wu[e].copy_(_storage_t(u, w.dtype))
            del u
            dn = _normal(rng, (w.F, w.d), inv)
            wd[e].copy_(_storage_t(dn, w.dtype))

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(w.E)))
        out.update(w_gate=wg, w_up=wu, w_down=wd)
    else:
        out.update(w_gate=None, w_up=None, w_down=None)

    rng = np.random.default_rng(ss[w.E + 1])
    if w.gen == "normal":
        x = _normal(rng, (w.T, w.d))
    elif w.gen == "zipf":
        V = w.zipf_vocab
        p = np.arange(1, V + 1, dtype=np.float64) ** (-w.zipf_s)
        p /= p.sum()
        ids = rng.choice(V, size=w.T, p=p)
        C = _normal(rng, (V, w.d))
        z = _normal(rng, (w.T, w.d))
        a = np.float32(w.zipf_alpha)
        x = (z + a * C[ids]) / np.float32(math.sqrt(1.0 + float(a) * float(a)))
        out["token_ids"] = torch.from_numpy(ids.astype(np.int64))
        del C, z
    else:
        raise ValueError(w.gen)
    out["x"] = _storage(x, w.dtype)
    return out


def random_small(T, d, E, k, F, cf, dtype, seed, gen="normal") -> tuple[Workload, dict]:
    """A small custom workload (parity cases that span several tiles and a ragged tail)."""
    w = Workload(f"custom_T{T}_d{d}_E{E}_k{k}_F{F}_{dtype}", T=T, d=d, E=E, k=k, F=F,
                 cf=cf, dtype=dtype, seed=seed, gen=gen, zipf_vocab=64)
    return w, generate(w)
