"""ctypes front end of the GPT-2 training-step oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it, and it
imports nothing from the GPU library.

Parity status of each oracle function (pins live in tests/test_oracle_pins.py and
tests/test_sampling.py): every forward layer, every backward formula, the AdamW
update and top-k sampling are pinned (closed forms, printed integers, invariants,
central finite differences and an independent autograd cross-check); nothing here
is "parity unpinned" (token batches and the layer order of weight files are pinned in
tests/test_io.py).  Incremental generation has no function of its own here: the
next-token logits after a prefix are the forward pass's logits at the prefix's last
position.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gpt2_oracle.cpp")
LIB = os.path.join(HERE, "libgpt2_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libgpt2_oracle.so with g++ and OpenMP."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c++17",
           "-Wall", SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        i64, i32, dbl, vp, cp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_char_p
        L.orc_last_error.restype = cp
        L.orc_num_parameters.argtypes = [i32] * 5
        L.orc_num_parameters.restype = i64
        L.orc_num_activations.argtypes = [i32] * 7
        L.orc_num_activations.restype = i64
        L.orc_create.argtypes = [i32] * 8
        L.orc_create.restype = vp
        L.orc_destroy.argtypes = [vp]
        L.orc_set_vec.argtypes = [vp, cp, vp, i64]
        L.orc_set_vec_f32.argtypes = [vp, cp, vp, i64]
        L.orc_get_vec.argtypes = [vp, cp, vp, i64]
        L.orc_act_numel.argtypes = [vp, cp, i32]
        L.orc_act_numel.restype = i64
        L.orc_get_act.argtypes = [vp, cp, i32, vp, i64]
        L.orc_forward.argtypes = [vp, vp, vp]
        L.orc_forward.restype = dbl
        L.orc_backward.argtypes = [vp]
        L.orc_adamw.argtypes = [vp, dbl, dbl, dbl, dbl, dbl, i32]
        L.orc_create_block.argtypes = [ctypes.c_int] * 9
        L.orc_create_block.restype = vp
        L.orc_num_parameters_block.argtypes = [ctypes.c_int] * 6
        L.orc_num_parameters_block.restype = i64
        L.orc_silu.argtypes = [vp, vp, i64]
        L.orc_silu.restype = None
        L.orc_silu_grad.argtypes = [vp, vp, i64]
        L.orc_silu_grad.restype = None
        L.orc_set_rotary.argtypes = [vp, ctypes.c_int, ctypes.c_double]
        L.orc_rope.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_double, ctypes.c_int]
        L.orc_rope.restype = None
        L.orc_gelu.argtypes = [vp, vp, i64]
        L.orc_gelu_grad.argtypes = [vp, vp, i64]
        L.orc_num_threads.restype = i32
        L.orc_set_mx.argtypes = [vp, ctypes.c_int]
        L.orc_mx_roundtrip.argtypes = [vp, vp, i64, ctypes.c_int]
        L.orc_mx_roundtrip.restype = None
        L.orc_matmul_backward_input_mx.argtypes = [vp, vp, i64, ctypes.c_int, ctypes.c_int, vp]
        L.orc_matmul_backward_input_mx.restype = None
        L.orc_set_num_threads.argtypes = [i32]
        L.orc_set_num_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_parameters(m) -> int:
    block = {"gpt2": 0, "llama": 1}[getattr(m, "block", "gpt2")]
    return int(lib().orc_num_parameters_block(m.vocab_size, m.max_seq_len, m.num_layers, m.num_heads, m.channels,
                                              block))


def silu(x) -> np.ndarray:
    """silu(x) = x sigmoid(x), the gate of the Llama-style block's SwiGLU MLP."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().orc_silu(_ptr(x), _ptr(y), x.size)
    return y


def silu_grad(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().orc_silu_grad(_ptr(x), _ptr(y), x.size)
    return y


def num_activations(m, B: int, T: int) -> int:
    return int(lib().orc_num_activations(m.vocab_size, m.max_seq_len, m.num_layers, m.num_heads, m.channels, B, T))


def gelu(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().orc_gelu(_ptr(x), _ptr(y), x.size)
    return y


def rope(x, pos, base: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotary position embedding of head vectors x [rows, hs] at positions pos [rows]
    (float64; see orc_rope)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, hs = x.shape
    p = np.ascontiguousarray(pos, dtype=np.int32).reshape(rows)
    y = np.empty_like(x)
    lib().orc_rope(_ptr(x), _ptr(y), rows, hs, _ptr(p), float(base), 1 if inverse else 0)
    return y


def gelu_grad(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().orc_gelu_grad(_ptr(x), _ptr(y), x.size)
    return y


def mx_roundtrip(x) -> np.ndarray:
    """x [rows, K] rounded to bf16, MX-encoded in blocks of 32 along K and decoded
    (float64; the operand an MX-mode product multiplies)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, K = x.shape
    y = np.empty_like(x)
    lib().orc_mx_roundtrip(_ptr(x), _ptr(y), rows, K)
    return y


def matmul_backward_input_mx(dout, w) -> np.ndarray:
    """dinp = dout [N, OC] w [OC, IC] with both operands through bf16 and the MX
    encoding in blocks of 32 along OC (dout's rows, and the columns of w)."""
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    N, OC = dout.shape
    OC2, IC = w.shape
    assert OC == OC2
    y = np.empty((N, IC), np.float64)
    lib().orc_matmul_backward_input_mx(_ptr(dout), _ptr(w), N, IC, OC, _ptr(y))
    return y


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the oracle's later calls (results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


class Oracle:
    """One oracle model instance: parameters, AdamW state and the plain activation set.

    prec: "f64" (the parity reference) or "f32" (the fp32 CPU trainer).
    """

    def __init__(self, m, B: int, T: int, prec: str = "f64"):
        self.m, self.B, self.T = m, B, T
        p = {"f32": 0, "f64": 1}[prec]
        block = {"gpt2": 0, "llama": 1}[getattr(m, "block", "gpt2")]
        h = lib().orc_create_block(p, m.vocab_size, m.max_seq_len, m.num_layers, m.num_heads, m.channels, B, T, block)
        if not h:
            raise ValueError(lib().orc_last_error().decode())
        self.h = h
        self.n_params = num_parameters(m)

    def close(self):
        if self.h:
            lib().orc_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set(self, name: str, values):
        a = np.asarray(values)
        if a.dtype == np.float32:
            a = np.ascontiguousarray(a)
            rc = lib().orc_set_vec_f32(self.h, name.encode(), _ptr(a), a.size)
        else:
            a = np.ascontiguousarray(a, dtype=np.float64)
            rc = lib().orc_set_vec(self.h, name.encode(), _ptr(a), a.size)
        if rc:
            raise ValueError(lib().orc_last_error().decode())

    def get(self, name: str) -> np.ndarray:
        out = np.empty(self.n_params, dtype=np.float64)
        if lib().orc_get_vec(self.h, name.encode(), _ptr(out), out.size):
            raise ValueError(lib().orc_last_error().decode())
        return out

    def act(self, name: str, layer: int = 0) -> np.ndarray:
        n = lib().orc_act_numel(self.h, name.encode(), layer)
        if n < 0:
            raise KeyError(f"{name}[{layer}]")
        out = np.empty(n, dtype=np.float64)
        if lib().orc_get_act(self.h, name.encode(), layer, _ptr(out), n):
            raise ValueError(lib().orc_last_error().decode())
        return out

    def forward(self, inputs, targets=None) -> float:
        inp = np.ascontiguousarray(inputs, dtype=np.int32)
        assert inp.size == self.B * self.T
        tgt = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32)
        loss = lib().orc_forward(self.h, _ptr(inp), None if tgt is None else _ptr(tgt))
        if loss != loss:
            raise ValueError(lib().orc_last_error().decode())
        return float(loss)

    def set_rotary(self, on: bool = True, base: float = 10000.0):
        """Rotary position embedding (RoFormer) instead of the learned wpe."""
        if lib().orc_set_rotary(self.h, 1 if on else 0, float(base)):
            raise ValueError(lib().orc_last_error().decode())

    def set_mx(self, on=True):
        """MX FP8 operands (bf16 values through the E4M3 / E8M0 block encoding) for the
        forward pass's block and lm_head products (on = True or 1), and with on = 2 also
        for the backward pass's input-gradient products of the same layers; the weight
        gradients keep the plain operands (straight-through)."""
        mode = int(on) if not isinstance(on, bool) else (1 if on else 0)
        if lib().orc_set_mx(self.h, mode):
            raise ValueError(lib().orc_last_error().decode())

    def backward(self):
        if lib().orc_backward(self.h):
            raise RuntimeError(lib().orc_last_error().decode())

    def adamw(self, lr, beta1, beta2, eps, weight_decay, step: int):
        if lib().orc_adamw(self.h, lr, beta1, beta2, eps, weight_decay, step):
            raise ValueError(lib().orc_last_error().decode())

    def step(self, inputs, targets, w, t: int) -> float:
        """forward + backward + AdamW with the workload's hyper-parameters; returns the loss."""
        loss = self.forward(inputs, targets)
        self.backward()
        self.adamw(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
        return loss


def sample_topk(logits, k: int, temperature: float, u: float) -> int:
    """Top-k sampling of one row ("GPT-2 from scratch with torch", 生成样本): keep the k
    highest logits (equal logits: the lower token id first), turn them into
    probabilities with a softmax at the given temperature, and draw by inverse
    transform with the caller's uniform u in [0, 1): the first kept token, in
    descending order, whose cumulative probability exceeds u."""
    z = np.asarray(logits, dtype=np.float64).reshape(-1)
    z = np.where(np.isnan(z), -np.inf, z)
    order = np.lexsort((np.arange(z.size), -z))[:min(k, z.size)]  # by -z, then by id
    top = z[order]
    if not np.isfinite(top[0]):
        return int(order[0])
    w = np.exp((top - top[0]) / float(temperature))
    cum = np.cumsum(w)
    i = int(np.searchsorted(cum, float(np.float32(u)) * cum[-1], side="right"))
    return int(order[min(i, order.size - 1)])


def token_batch(ids, B: int, T: int, i: int):
    """Batch i of a token stream ("1000 行 C 代码完成 GPT-2 训练的 LLM.c", 快速开始吧: a raw
    int32 id stream): the B*T + 1 ids from i*B*T on, the stream read as a circle; inputs
    are the first B*T, targets the next B*T, both [B, T].  There are len(ids) // (B*T)
    batches."""
    ids = np.asarray(ids, dtype=np.int32)
    n, bt = ids.size, B * T
    if not 0 <= i < n // bt:
        raise IndexError(i)
    win = ids[(i * bt + np.arange(bt + 1)) % n]
    return win[:-1].reshape(B, T), win[1:].reshape(B, T)


def lexicographic_layer_order(L: int):
    """The layers as a weight file that sorts them by name stores them
    ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン", 重みの読み込み): by the text of
    the decimal index."""
    return sorted(range(L), key=str)


def permute_layers(m, params, to_lexicographic: bool):
    """A flat parameter array (layer-major: wte, wpe, the layer blocks, ln_f) with its
    layer blocks moved between numeric and lexicographic layer order."""
    C, L = m.channels, m.num_layers
    head = (m.vocab_size + m.max_seq_len) * C
    block = 12 * C * C + 13 * C
    p = np.asarray(params)
    blocks = [p[head + l * block: head + (l + 1) * block] for l in range(L)]
    order = lexicographic_layer_order(L)
    if to_lexicographic:
        new = [blocks[l] for l in order]
    else:
        new = [None] * L
        for k, l in enumerate(order):
            new[l] = blocks[k]
    return np.concatenate([p[:head]] + new + [p[head + L * block:]])
