"""Seeded synthetic inputs shared by the oracle-side tests and the GPU harness.

This module holds no arithmetic of the model itself: it only draws numbers.
Both sides of every parity check receive the very same bytes from here.

Generators (published definitions, re-implemented here):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014).  Output i (0-based) of the stream with seed s is
  ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` with the published two-multiply
  finaliser, so it is counter based: any element can be drawn on its own.
* 53-bit uniforms in [0, 1): the top 53 bits of a SplitMix64 output times 2^-53.
* Normals by the Box-Muller transform (Box & Muller 1958), in float64:
  normal i = sqrt(-2 ln(1 - u_{2i})) * cos(2 pi u_{2i+1}), then rounded to fp32.
* Zipf token ids: P(id = k) proportional to (k + 1)^-s over [0, V), drawn by
  inverse-CDF search on a float64 cumulative table.

The pages do not specify an initialisation ("GPT-2 from scratch with torch",
section "输出" says weight initialisation is skipped); the recipe used here is
N(0, 0.02) for embeddings and the qkv/fc weights, N(0, 0.02/sqrt(2L)) for the
two residual-output projections, LayerNorm gamma = 1, beta = 0, all biases 0,
and the lm_head tied to the token embedding.
"""
from __future__ import annotations

import dataclasses
import math

import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

PARAM_SEED = 1337
TOKEN_SEED = 42


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """GPT-2 hyper-parameters, named as in the llm.c run banner
    (max_seq_len, vocab_size, num_layers, num_heads, channels)."""

    max_seq_len: int
    vocab_size: int
    num_layers: int
    num_heads: int
    channels: int
    block: str = "gpt2"   # "gpt2", or "llama": RMSNorm, no biases, SwiGLU MLP, rotary positions


def llama_hidden(C: int) -> int:
    """SwiGLU width of the Llama-style block: 8C/3 rounded up to a multiple of 64."""
    return 64 * ((C + 23) // 24)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic training workload: model shape, batch, precision, tokens."""

    name: str
    model: ModelShape
    B: int
    T: int
    dtype: str            # "fp32" or "bf16" (bf16 weights/activations, fp32 master state)
    tokens: str           # "uniform" or "zipf"
    zipf_s: float = 1.1
    index: int = 0        # offsets the token seed so workloads draw different ids
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


GPT2_TINY_CHAR = ModelShape(32, 65, 2, 4, 64)
GPT2_124M = ModelShape(1024, 50257, 12, 12, 768)
GPT2_350M = ModelShape(1024, 50257, 24, 16, 1024)
GPT2_1558M = ModelShape(1024, 50257, 48, 25, 1600)
# a Llama-style model of GPT-2 124M's size (C 768, 12 layers, 12 heads, SwiGLU width 2048)
LLAMA_124M = ModelShape(1024, 50257, 12, 12, 768, "llama")

WORKLOADS = {
    "tiny_char_b4t32_fp32": Workload("tiny_char_b4t32_fp32", GPT2_TINY_CHAR, 4, 32, "fp32", "uniform", index=0),
    "gpt2_124m_b4t64_fp32": Workload("gpt2_124m_b4t64_fp32", GPT2_124M, 4, 64, "fp32", "uniform", index=1),
    "gpt2_124m_b8t1024_bf16": Workload("gpt2_124m_b8t1024_bf16", GPT2_124M, 8, 1024, "bf16", "uniform", index=2),
    "gpt2_350m_b8t1024_bf16_zipf": Workload("gpt2_350m_b8t1024_bf16_zipf", GPT2_350M, 8, 1024, "bf16", "zipf", index=3),
    "gpt2_1558m_b4t1024_bf16": Workload("gpt2_1558m_b4t1024_bf16", GPT2_1558M, 4, 1024, "bf16", "uniform", index=4),
    "llama_124m_b8t1024_bf16": Workload("llama_124m_b8t1024_bf16", LLAMA_124M, 8, 1024, "bf16", "uniform", index=5),
}


# --------------------------------------------------------------------------- generators

def splitmix64(seed: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs number ``idx`` (uint64 array, 0-based) of stream ``seed``."""
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (idx.astype(np.uint64) + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform53(seed: int, idx: np.ndarray) -> np.ndarray:
    """Float64 uniforms in [0, 1) from the top 53 bits of SplitMix64 output ``idx``."""
    return (splitmix64(seed, idx) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, idx: np.ndarray) -> np.ndarray:
    """Float64 standard normals; normal ``i`` consumes uniforms 2i and 2i+1."""
    idx = idx.astype(np.uint64)
    u1 = uniform53(seed, idx * np.uint64(2))
    u2 = uniform53(seed, idx * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)


# --------------------------------------------------------------------------- parameters

def param_tensors(m: ModelShape):
    """(name, numel, init) for every parameter tensor in the flat order.

    The order is layer-major, following the module tree (wte, wpe, then per
    block ln_1, attn.c_attn, attn.c_proj, ln_2, mlp.c_fc, mlp.c_proj, then
    ln_f); weights are (out, in) row-major.  ``init`` is ("normal", std),
    ("const", value).
    """
    C, L = m.channels, m.num_layers
    std = 0.02
    std_res = 0.02 / math.sqrt(2 * L)
    out = [("wte", m.vocab_size * C, ("normal", std)),
           ("wpe", m.max_seq_len * C, ("normal", std))]
    if m.block == "llama":
        # RMSNorm gains, no biases; gate|up interleaved by row (2j gate, 2j+1 up); wpe unused
        H = llama_hidden(C)
        for l in range(L):
            out += [
                (f"h{l}.rms1.w", C, ("const", 1.0)),
                (f"h{l}.qkv.w", 3 * C * C, ("normal", std)),
                (f"h{l}.proj.w", C * C, ("normal", std_res)),
                (f"h{l}.rms2.w", C, ("const", 1.0)),
                (f"h{l}.gateup.w", 2 * H * C, ("normal", std)),
                (f"h{l}.down.w", C * H, ("normal", std_res)),
            ]
        out += [("rmsf.w", C, ("const", 1.0))]
        return out
    for l in range(L):
        out += [
            (f"h{l}.ln1.w", C, ("const", 1.0)),
            (f"h{l}.ln1.b", C, ("const", 0.0)),
            (f"h{l}.qkv.w", 3 * C * C, ("normal", std)),
            (f"h{l}.qkv.b", 3 * C, ("const", 0.0)),
            (f"h{l}.proj.w", C * C, ("normal", std_res)),
            (f"h{l}.proj.b", C, ("const", 0.0)),
            (f"h{l}.ln2.w", C, ("const", 1.0)),
            (f"h{l}.ln2.b", C, ("const", 0.0)),
            (f"h{l}.fc.w", 4 * C * C, ("normal", std)),
            (f"h{l}.fc.b", 4 * C, ("const", 0.0)),
            (f"h{l}.fcproj.w", C * 4 * C, ("normal", std_res)),
            (f"h{l}.fcproj.b", C, ("const", 0.0)),
        ]
    out += [("lnf.w", C, ("const", 1.0)), ("lnf.b", C, ("const", 0.0))]
    return out


def param_offsets(m: ModelShape):
    """name -> (offset, numel) in the flat parameter vector."""
    offs, o = {}, 0
    for name, n, _ in param_tensors(m):
        offs[name] = (o, n)
        o += n
    return offs


def num_parameters(m: ModelShape) -> int:
    return sum(n for _, n, _ in param_tensors(m))


def init_params(m: ModelShape, seed: int = PARAM_SEED, chunk: int = 1 << 22) -> np.ndarray:
    """The flat fp32 parameter vector.  Element i of a normal-initialised tensor
    is std * normal(seed, i) with i the flat index, so any slice is reproducible
    on its own (chunks are filled by a thread pool; the result does not depend on
    the order)."""
    import concurrent.futures
    total = num_parameters(m)
    out = np.empty(total, dtype=np.float32)
    jobs = []
    o = 0
    for _, n, (kind, val) in param_tensors(m):
        if kind == "const":
            out[o:o + n] = val
        else:
            for s in range(0, n, chunk):
                jobs.append((o + s, o + min(n, s + chunk), val))
        o += n

    def fill(job):
        b, e, val = job
        out[b:e] = (val * normal(seed, np.arange(b, e, dtype=np.uint64))).astype(np.float32)

    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, jobs))
    return out


# --------------------------------------------------------------------------- tokens

def zipf_cdf(V: int, s: float) -> np.ndarray:
    w = (np.arange(V, dtype=np.float64) + 1.0) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def token_windows(w: Workload, seed: int | None = None, B: int | None = None, T: int | None = None) -> np.ndarray:
    """int32 [B, T+1] token windows; inputs are [:, :T], targets [:, 1:]."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    seed = TOKEN_SEED + w.index if seed is None else seed
    V = w.model.vocab_size
    u = uniform53(seed, np.arange(B * (T + 1), dtype=np.uint64))
    if w.tokens == "uniform":
        ids = np.minimum(np.floor(u * V), V - 1).astype(np.int32)
    elif w.tokens == "zipf":
        ids = np.searchsorted(zipf_cdf(V, w.zipf_s), u, side="right").astype(np.int32)
        ids = np.minimum(ids, V - 1)
    else:
        raise ValueError(w.tokens)
    return ids.reshape(B, T + 1)


def inputs_targets(w: Workload, **kw):
    win = token_windows(w, **kw)
    return np.ascontiguousarray(win[:, :-1]), np.ascontiguousarray(win[:, 1:])
