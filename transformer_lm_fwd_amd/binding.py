"""ctypes binding of the gfx950 GPT-2 training-step library (include/gpt2.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libgpt2_hip.so.  PyTorch supplies the device arena (one uint8 tensor) and the
stream.  If the library has not been built this module raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GPT2_HIP_LIB may name another build of the same library (e.g. to compare two builds).
LIB_PATH = os.environ.get("GPT2_HIP_LIB") or os.path.join(HERE, "_lib", "libgpt2_hip.so")

GPT2_FP32, GPT2_BF16 = 0, 1
STATUS = {0: "GPT2_OK", -1: "GPT2_E_INVAL", -2: "GPT2_E_SIZE", -3: "GPT2_E_ALIGN", -4: "GPT2_E_STATE",
          -5: "GPT2_E_HIP"}

# tensor ids (enum gpt2_tensor_id)
T_PARAMS, T_GRADS, T_ADAM_M, T_ADAM_V, T_PARAMS_BF16 = 0, 1, 2, 3, 4
T_ENCODED, T_LNF, T_LNF_STATS, T_LOGITS, T_LOSSES, T_LOSS = 5, 6, 7, 8, 9, 10
T_LN1, T_LN1_STATS, T_QKV, T_ATTY, T_ATT_LSE, T_RESIDUAL2 = 16, 17, 18, 19, 20, 21
T_LN2, T_LN2_STATS, T_FCH, T_FCH_GELU, T_RESIDUAL3 = 22, 23, 24, 25, 26

EXPORTS = ("gpt2_alloc_arena", "gpt2_free_arena", "gpt2_sync_weights", "gpt2_forward", "gpt2_backward",
           "gpt2_adamw_step", "gpt2_backward_adamw", "gpt2_tensor_info", "gpt2_num_parameters", "gpt2_profile",
           "gpt2_profile_read", "gpt2_profile_order", "gpt2_set_side_stream", "gpt2_eval_loss", "gpt2_mx_weight_codes", "gpt2_gen_alloc", "gpt2_gen_free", "gpt2_gen_length", "gpt2_gen_prefill",
           "gpt2_gen_decode", "gpt2_sample_topk", "gpt2_tokens_count", "gpt2_tokens_batch",
           "gpt2_params_permute", "gpt2_checkpoint_write", "gpt2_checkpoint_read", "gpt2_set_position_encoding",
           "gpt2_num_parameters_block", "gpt2_alloc_arena_block",
           "gpt2_mx_attach",
           "gpt2_set_gemm_format", "gpt2_mx_buffer", "gpt2_mx_quantize", "gpt2_mx_gemm", "gpt2_mfma_peak", "gpt2_gen_decode_noalloc",
           "gpt2_last_error")
GPT2_ORDER_NUMERIC, GPT2_ORDER_LEXICOGRAPHIC = 0, 1
GPT2_GEMM_BF16, GPT2_GEMM_MXFP8, GPT2_GEMM_MXFP8_DX = 0, 1, 2
GPT2_POS_LEARNED, GPT2_POS_ROTARY = 0, 1
GPT2_BLOCK_GPT2, GPT2_BLOCK_LLAMA = 0, 1
GPT2_EPI_BIAS, GPT2_EPI_BIAS_RES, GPT2_EPI_BIAS_GELU, GPT2_EPI_GELU_BWD = 0, 1, 2, 3
GPT2_MX_BUF_INPUT, GPT2_MX_BUF_GELU, GPT2_MX_BUF_DY = 0, 1, 2


class gpt2_config(ctypes.Structure):
    _fields_ = [("max_seq_len", ctypes.c_int32), ("vocab_size", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("channels", ctypes.c_int32)]


class gpt2_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class Gpt2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib():
    """Loads libgpt2_hip.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m transformer_lm_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        cfgp = ctypes.POINTER(gpt2_config)
        L.gpt2_alloc_arena.argtypes = [cfgp, i32, i32, i32, vp, sz, ctypes.POINTER(sz), ctypes.POINTER(vp)]
        L.gpt2_free_arena.argtypes = [vp]
        L.gpt2_sync_weights.argtypes = [vp, vp]
        L.gpt2_forward.argtypes = [vp, vp, vp, vp]
        L.gpt2_backward.argtypes = [vp, vp]
        L.gpt2_adamw_step.argtypes = [vp, f32, f32, f32, f32, f32, i32, vp]
        L.gpt2_backward_adamw.argtypes = [vp, f32, f32, f32, f32, f32, i32, vp]
        L.gpt2_tensor_info.argtypes = [vp, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(i64), ctypes.POINTER(i64),
                                       ctypes.POINTER(i64), ctypes.POINTER(i32)]
        L.gpt2_num_parameters.argtypes = [cfgp]
        L.gpt2_num_parameters.restype = i64
        L.gpt2_last_error.restype = ctypes.c_char_p
        L.gpt2_profile.argtypes = [ctypes.c_int]
        L.gpt2_profile_read.argtypes = [ctypes.POINTER(gpt2_kernel_stat), i32, ctypes.POINTER(i32)]
        L.gpt2_profile_order.argtypes = [ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
        L.gpt2_set_side_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.gpt2_eval_loss.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, i32, ctypes.c_void_p,
                                     ctypes.c_void_p]
        L.gpt2_mfma_peak.argtypes = [i32, ctypes.POINTER(ctypes.c_double), vp]
        L.gpt2_gen_alloc.argtypes = [vp, i32, i32, vp, sz, ctypes.POINTER(sz), ctypes.POINTER(vp)]
        L.gpt2_gen_free.argtypes = [vp]
        L.gpt2_gen_length.argtypes = [vp]
        L.gpt2_gen_prefill.argtypes = [vp, vp, i32, vp, vp]
        L.gpt2_gen_decode.argtypes = [vp, vp, vp, vp]
        L.gpt2_gen_decode_noalloc.argtypes = [vp, vp, vp, vp]
        L.gpt2_sample_topk.argtypes = [vp, i32, i32, i64, i32, f32, vp, vp]
        cp = ctypes.c_char_p
        L.gpt2_tokens_count.argtypes = [cp]
        L.gpt2_tokens_count.restype = i64
        L.gpt2_tokens_batch.argtypes = [cp, i32, i32, i64, vp, vp]
        L.gpt2_params_permute.argtypes = [cfgp, vp, vp, i32, i32]
        L.gpt2_checkpoint_write.argtypes = [cp, cfgp, i32, vp, vp, vp]
        L.gpt2_checkpoint_read.argtypes = [cp, cfgp, ctypes.POINTER(i32), vp, vp, vp, ctypes.POINTER(i32)]
        L.gpt2_set_position_encoding.argtypes = [vp, i32, f32, vp]
        L.gpt2_num_parameters_block.argtypes = [cfgp, i32]
        L.gpt2_num_parameters_block.restype = i64
        L.gpt2_alloc_arena_block.argtypes = [cfgp, i32, i32, i32, i32, vp, sz, ctypes.POINTER(sz), ctypes.POINTER(vp)]
        L.gpt2_mx_attach.argtypes = [vp, vp, sz, ctypes.POINTER(sz)]
        L.gpt2_set_gemm_format.argtypes = [vp, i32]
        L.gpt2_mx_buffer.argtypes = [vp, i32, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
        L.gpt2_mx_weight_codes.argtypes = [vp, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(sz), ctypes.POINTER(i64),
                                           ctypes.POINTER(i64)]
        L.gpt2_mx_quantize.argtypes = [vp, i64, i32, i32, vp, i64, vp, vp]
        L.gpt2_mx_gemm.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, i32, i32, i32, i32, vp, vp, vp, vp]
        for name in EXPORTS:
            if name not in ("gpt2_num_parameters", "gpt2_num_parameters_block", "gpt2_last_error", "gpt2_tokens_count"):
                L[name].restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise Gpt2Error(rc, lib().gpt2_last_error().decode())


def make_config(m) -> gpt2_config:
    return gpt2_config(m.max_seq_len, m.vocab_size, m.num_layers, m.num_heads, m.channels)


def block_of(m) -> int:
    """GPT2_BLOCK_* of a model shape (its `block` field: "gpt2" or "llama")."""
    return {"gpt2": GPT2_BLOCK_GPT2, "llama": GPT2_BLOCK_LLAMA}[getattr(m, "block", "gpt2")]


def num_parameters(m) -> int:
    return int(lib().gpt2_num_parameters_block(ctypes.byref(make_config(m)), block_of(m)))


def arena_bytes(m, B: int, T: int, dtype: int) -> int:
    need = ctypes.c_size_t(0)
    _check(lib().gpt2_alloc_arena_block(ctypes.byref(make_config(m)), block_of(m), B, T, dtype, None, 0,
                                        ctypes.byref(need), None))
    return int(need.value)


def profile(enable: bool) -> None:
    """Starts (clearing earlier records) or stops the library's launch profiler."""
    _check(lib().gpt2_profile(1 if enable else 0))


def profile_read():
    """Per-kernel aggregates of the recorded launches (waits for their events):
    a list of dicts with name, launches, total_ms, flops, bytes."""
    n = ctypes.c_int32(0)
    _check(lib().gpt2_profile_read(None, 0, ctypes.byref(n)))
    arr = (gpt2_kernel_stat * max(1, n.value))()
    _check(lib().gpt2_profile_read(arr, n.value, ctypes.byref(n)))
    return [dict(name=r.name.decode(), launches=int(r.launches), total_ms=float(r.total_ms), flops=float(r.flops),
                 bytes=float(r.bytes)) for r in arr[:n.value]]


def profile_order():
    """Kernel names of the recorded launches in launch order (one entry per dispatch)."""
    names = [s["name"] for s in profile_read()]
    n = ctypes.c_int32(0)
    _check(lib().gpt2_profile_order(None, 0, ctypes.byref(n)))
    arr = (ctypes.c_int32 * max(1, n.value))()
    _check(lib().gpt2_profile_order(arr, n.value, ctypes.byref(n)))
    return [names[i] for i in arr[:n.value]]


MFMA_BF16_32X32X16, MFMA_BF16_16X16X32, MFMA_MXFP8_32X32X64 = 0, 1, 2


def mfma_peak(kind: int = MFMA_BF16_32X32X16, stream=None) -> float:
    """Sustained TFLOP/s of one MFMA form over the whole chip (gpt2_mfma_peak)."""
    out = ctypes.c_double(0.0)
    _check(lib().gpt2_mfma_peak(int(kind), ctypes.byref(out), _stream_ptr(stream)))
    return float(out.value)


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Arena:
    """One arena on the current CUDA (HIP) device: parameters, AdamW state,
    activations and scratch in one zero-filled torch uint8 buffer."""

    def __init__(self, m, B: int, T: int, dtype: str = "bf16", device="cuda"):
        import torch
        self.m, self.B, self.T = m, B, T
        self.dtype = {"fp32": GPT2_FP32, "bf16": GPT2_BF16}[dtype]
        self.dtype_name = dtype
        self.nbytes = arena_bytes(m, B, T, self.dtype)
        self.buf = torch.zeros(self.nbytes + 256, dtype=torch.uint8, device=device)
        pad = (-self.buf.data_ptr()) % 256
        self.base = self.buf[pad:pad + self.nbytes]
        h = ctypes.c_void_p()
        _check(lib().gpt2_alloc_arena_block(ctypes.byref(make_config(m)), block_of(m), B, T, self.dtype,
                                            ctypes.c_void_p(self.base.data_ptr()), self.nbytes, None,
                                            ctypes.byref(h)))
        self.h = h
        # the second stream of the forward and backward passes comes from torch
        # (default priority), like the memory
        self.side_stream = torch.cuda.Stream(device=self.buf.device)
        _check(lib().gpt2_set_side_stream(self.h, ctypes.c_void_p(self.side_stream.cuda_stream)))
        self.n_params = num_parameters(m)
        self._inputs = None
        self._targets = None

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_free_arena(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ tensors
    def info(self, tensor_id: int, layer: int = 0):
        off, rows, cols, ld, dt = ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib().gpt2_tensor_info(self.h, tensor_id, layer, ctypes.byref(off), ctypes.byref(rows),
                                      ctypes.byref(cols), ctypes.byref(ld), ctypes.byref(dt)))
        return off.value, rows.value, cols.value, ld.value, dt.value

    def tensor(self, tensor_id: int, layer: int = 0):
        """A torch view of an arena tensor, shape [rows, row_stride] narrowed to [rows, cols]."""
        import torch
        off, rows, cols, ld, dt = self.info(tensor_id, layer)
        tdt, es = (torch.float32, 4) if dt == GPT2_FP32 else (torch.bfloat16, 2)
        raw = self.base[off:off + rows * ld * es].view(tdt).view(rows, ld)
        return raw[:, :cols]

    # ------------------------------------------------------------------ steps
    def load_params(self, params, stream=None):
        """Copies a flat fp32 parameter vector into the master weights and refreshes derived copies."""
        import torch
        p = torch.as_tensor(params, dtype=torch.float32)
        assert p.numel() == self.n_params, (p.numel(), self.n_params)
        self.tensor(T_PARAMS).view(-1).copy_(p.view(-1))
        _check(lib().gpt2_sync_weights(self.h, _stream_ptr(stream)))

    def _ids(self, x):
        import torch
        t = torch.as_tensor(x)
        if t.dtype != torch.int32:
            t = t.to(torch.int32)
        if tuple(t.shape) != (self.B, self.T):
            raise ValueError(f"token array must have shape {(self.B, self.T)}, got {tuple(t.shape)}")
        lo, hi = int(t.min()), int(t.max())
        if lo < 0 or hi >= self.m.vocab_size:
            raise ValueError(f"token ids must lie in [0, {self.m.vocab_size}), got [{lo}, {hi}]")
        return t.to(self.base.device).contiguous()

    def forward(self, inputs, targets=None, stream=None, check_ids=True):
        """check_ids=False skips the host-side id range check (which synchronises);
        then inputs/targets must already be int32 device tensors of shape (B, T)."""
        # keep the device token arrays alive for the backward pass
        if check_ids:
            self._inputs = self._ids(inputs)
            self._targets = None if targets is None else self._ids(targets)
        else:
            self._inputs, self._targets = inputs, targets
        _check(lib().gpt2_forward(self.h, ctypes.c_void_p(self._inputs.data_ptr()),
                                  None if self._targets is None else ctypes.c_void_p(self._targets.data_ptr()),
                                  _stream_ptr(stream)))

    def backward(self, stream=None):
        _check(lib().gpt2_backward(self.h, _stream_ptr(stream)))

    def adamw_step(self, lr, beta1, beta2, eps, weight_decay, step: int, stream=None):
        _check(lib().gpt2_adamw_step(self.h, lr, beta1, beta2, eps, weight_decay, step, _stream_ptr(stream)))

    def backward_adamw(self, lr, beta1, beta2, eps, weight_decay, step: int, stream=None):
        """gpt2_backward and gpt2_adamw_step fused (per-layer updates overlap the backward pass)."""
        _check(lib().gpt2_backward_adamw(self.h, lr, beta1, beta2, eps, weight_decay, step, _stream_ptr(stream)))

    def loss(self) -> float:
        return float(self.tensor(T_LOSS).item())

    def eval_loss(self, path: str, num_batches: int, first: int = 0, stream=None) -> float:
        """Mean forward loss over batches first .. first + num_batches - 1 of an int32
        token file (the validation loss of a training run; no backward pass): the
        batches are read on the host and the mean is taken by gpt2_eval_loss."""
        import torch
        xs, ys = zip(*(tokens_batch(path, self.B, self.T, i) for i in range(first, first + num_batches)))
        x = torch.stack([self._ids(v) for v in xs])
        y = torch.stack([self._ids(v) for v in ys])
        out = torch.empty(1, dtype=torch.float32, device=self.base.device)
        _check(lib().gpt2_eval_loss(self.h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                    num_batches, ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return float(out.item())

    # ------------------------------------------------------------------ checkpoints
    def save_checkpoint(self, path: str, step: int, moments: bool = True) -> None:
        """Master weights (and the AdamW moments) to a checkpoint file (gpt2_checkpoint_write)."""
        import numpy as np
        if block_of(self.m) != GPT2_BLOCK_GPT2:
            raise ValueError("checkpoint files describe GPT-2 arenas")
        p = self.tensor(T_PARAMS).cpu().numpy().reshape(-1)
        m = self.tensor(T_ADAM_M).cpu().numpy().reshape(-1) if moments else None
        v = self.tensor(T_ADAM_V).cpu().numpy().reshape(-1) if moments else None
        arrs = [np.ascontiguousarray(a, dtype=np.float32) if a is not None else None for a in (p, m, v)]
        _check(lib().gpt2_checkpoint_write(path.encode(), ctypes.byref(make_config(self.m)), step,
                                           *[a.ctypes.data if a is not None else None for a in arrs]))

    def load_checkpoint(self, path: str, stream=None) -> int:
        """Reads a checkpoint into the master weights (and moments, if the file has them),
        refreshes the bf16 copy, and returns the file's AdamW step."""
        import numpy as np
        import torch
        if block_of(self.m) != GPT2_BLOCK_GPT2:
            raise ValueError("checkpoint files describe GPT-2 arenas")
        n = self.n_params
        p, m, v = (np.empty(n, np.float32) for _ in range(3))
        step, has = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib().gpt2_checkpoint_read(path.encode(), ctypes.byref(make_config(self.m)), ctypes.byref(step),
                                          p.ctypes.data, m.ctypes.data, v.ctypes.data, ctypes.byref(has)))
        self.tensor(T_PARAMS).view(-1).copy_(torch.from_numpy(p))
        if has.value:
            self.tensor(T_ADAM_M).view(-1).copy_(torch.from_numpy(m))
            self.tensor(T_ADAM_V).view(-1).copy_(torch.from_numpy(v))
        _check(lib().gpt2_sync_weights(self.h, _stream_ptr(stream)))
        return int(step.value)

    def set_position_encoding(self, mode: int, base: float = 10000.0, stream=None) -> None:
        """GPT2_POS_LEARNED (wpe) or GPT2_POS_ROTARY (rotary q / k turns; base of the frequencies)."""
        _check(lib().gpt2_set_position_encoding(self.h, mode, base, _stream_ptr(stream)))

    # ------------------------------------------------------------------ MX FP8 products
    def set_gemm_format(self, fmt: int) -> None:
        """GPT2_GEMM_BF16, GPT2_GEMM_MXFP8 (forward products) or GPT2_GEMM_MXFP8_DX (and the
        backward pass's input-gradient products); the first switch to an MX format gives
        the arena its MX memory (a torch uint8 buffer on the same device)."""
        import torch
        if fmt in (GPT2_GEMM_MXFP8, GPT2_GEMM_MXFP8_DX) and getattr(self, "_mx", None) is None:
            need = ctypes.c_size_t(0)
            _check(lib().gpt2_mx_attach(self.h, None, 0, ctypes.byref(need)))
            buf = torch.empty(int(need.value) + 256, dtype=torch.uint8, device=self.base.device)
            pad = (-buf.data_ptr()) % 256
            _check(lib().gpt2_mx_attach(self.h, ctypes.c_void_p(buf.data_ptr() + pad), int(need.value), None))
            self._mx = buf
        _check(lib().gpt2_set_gemm_format(self.h, fmt))

    def mx_weight_codes(self, index: int, transposed: bool = False):
        """Views (codes [rows, ld] uint8, scales [ld / 128, rows, 4] uint8) of the MX codes
        of forward weight `index` or of its transpose (gpt2_mx_weight_codes)."""
        qo, so, rows, ld = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().gpt2_mx_weight_codes(self.h, index, 1 if transposed else 0, ctypes.byref(qo), ctypes.byref(so),
                                          ctypes.byref(rows), ctypes.byref(ld)))
        pad = (-self._mx.data_ptr()) % 256
        base = self._mx[pad:]
        r, k = rows.value, ld.value
        return (base[qo.value:qo.value + r * k].view(r, k),
                base[so.value:so.value + r * k // 32].view(k // 128, r, 4))

    def mx_buffer(self, which: int):
        """Views (codes [rows, ld] uint8, scales [ld / 128, rows, 4] uint8) of one of the
        arena's MX input buffers (gpt2_mx_buffer)."""
        qo, so, rows, ld = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().gpt2_mx_buffer(self.h, which, ctypes.byref(qo), ctypes.byref(so), ctypes.byref(rows),
                                    ctypes.byref(ld)))
        pad = (-self._mx.data_ptr()) % 256
        base = self._mx[pad:]
        r, k = rows.value, ld.value
        return (base[qo.value:qo.value + r * k].view(r, k),
                base[so.value:so.value + r * k // 32].view(k // 128, r, 4))

    def step(self, inputs, targets, w, t: int, check_ids=True, fused=True) -> None:
        """forward + backward + AdamW with a workload's hyper-parameters (fused: the
        AdamW update overlaps the backward pass; results are bitwise the same)."""
        self.forward(inputs, targets, check_ids=check_ids)
        if fused:
            self.backward_adamw(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)
        else:
            self.backward()
            self.adamw_step(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, t)


class Generator:
    """Incremental generation with a key/value cache over an Arena's parameters
    (bf16, head size 64): `batch` sequences of up to `max_len` tokens advancing
    together.  prefill / decode return the next-token logits as a device fp32
    tensor [batch, vocab_size]."""

    def __init__(self, arena: Arena, batch: int, max_len: int):
        import torch
        self.arena, self.batch, self.max_len = arena, batch, max_len
        need = ctypes.c_size_t(0)
        _check(lib().gpt2_gen_alloc(arena.h, batch, max_len, None, 0, ctypes.byref(need), None))
        self.nbytes = int(need.value)
        self.buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=arena.base.device)
        pad = (-self.buf.data_ptr()) % 256
        self.base = self.buf[pad:pad + self.nbytes]
        h = ctypes.c_void_p()
        _check(lib().gpt2_gen_alloc(arena.h, batch, max_len, ctypes.c_void_p(self.base.data_ptr()), self.nbytes,
                                    None, ctypes.byref(h)))
        self.h = h
        self.logits = torch.empty(batch, arena.m.vocab_size, dtype=torch.float32, device=arena.base.device)
        self._tok = None

    def close(self):
        if getattr(self, "h", None):
            lib().gpt2_gen_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def length(self) -> int:
        return int(lib().gpt2_gen_length(self.h))

    def _ids(self, x, shape):
        import torch
        t = torch.as_tensor(x)
        if t.dtype != torch.int32:
            t = t.to(torch.int32)
        if tuple(t.shape) != shape:
            raise ValueError(f"token array must have shape {shape}, got {tuple(t.shape)}")
        lo, hi = int(t.min()), int(t.max())
        if lo < 0 or hi >= self.arena.m.vocab_size:
            raise ValueError(f"token ids must lie in [0, {self.arena.m.vocab_size}), got [{lo}, {hi}]")
        return t.to(self.base.device).contiguous()

    def prefill(self, tokens, stream=None, check_ids=True):
        """tokens [batch, n]; returns the logits of position n - 1 (device fp32)."""
        t = self._ids(tokens, (self.batch, int(tokens.shape[1]))) if check_ids else tokens
        self._tok = t
        _check(lib().gpt2_gen_prefill(self.h, ctypes.c_void_p(t.data_ptr()), int(t.shape[1]),
                                      ctypes.c_void_p(self.logits.data_ptr()), _stream_ptr(stream)))
        return self.logits

    def decode(self, tokens, stream=None, check_ids=True):
        """tokens [batch] (the token at the current length); returns the next logits."""
        t = self._ids(tokens, (self.batch,)) if check_ids else tokens
        self._tok = t
        _check(lib().gpt2_gen_decode(self.h, ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(self.logits.data_ptr()),
                                     _stream_ptr(stream)))
        return self.logits


def sample_topk(logits, k: int, temperature: float, uniforms):
    """gpt2_sample_topk on host arrays: logits float32 [rows, V] (C-contiguous rows),
    uniforms float32 [rows] in [0, 1); returns int32 [rows]."""
    import numpy as np
    z = np.ascontiguousarray(logits, dtype=np.float32)
    if z.ndim != 2:
        raise ValueError("logits must be 2-D [rows, V]")
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(-1)
    if u.size != z.shape[0]:
        raise ValueError("one uniform per row is required")
    out = np.empty(z.shape[0], dtype=np.int32)
    _check(lib().gpt2_sample_topk(z.ctypes.data, z.shape[0], z.shape[1], z.shape[1], k, temperature, u.ctypes.data,
                                  out.ctypes.data))
    return out


def tokens_count(path: str) -> int:
    n = int(lib().gpt2_tokens_count(path.encode()))
    if n < 0:
        _check(n)
    return n


def tokens_batch(path: str, B: int, T: int, batch: int):
    """Batch `batch` of an int32 token file: (inputs, targets), int32 [B, T] each."""
    import numpy as np
    x = np.empty((B, T), np.int32)
    y = np.empty((B, T), np.int32)
    _check(lib().gpt2_tokens_batch(path.encode(), B, T, batch, x.ctypes.data, y.ctypes.data))
    return x, y


def params_permute(m, params, from_order: int, to_order: int):
    """A flat fp32 parameter array reordered between layer orders (gpt2_params_permute)."""
    import numpy as np
    src = np.ascontiguousarray(params, dtype=np.float32)
    dst = np.empty_like(src)
    _check(lib().gpt2_params_permute(ctypes.byref(make_config(m)), src.ctypes.data, dst.ctypes.data, from_order,
                                     to_order))
    return dst


def mx_quantize(x, stream=None):
    """MX FP8 quantization (gpt2_mx_quantize) of a device bf16 tensor [rows, K]:
    returns (codes uint8 [rows, Kp], scales uint8 [Kp / 128, rows, 4]), Kp = K rounded up to 128."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    R, K = x.shape
    Kp = (K + 127) // 128 * 128
    q = torch.empty(R, Kp, dtype=torch.uint8, device=x.device)
    sc = torch.empty(Kp // 128, R, 4, dtype=torch.uint8, device=x.device)
    _check(lib().gpt2_mx_quantize(ctypes.c_void_p(x.data_ptr()), x.stride(0), R, K, ctypes.c_void_p(q.data_ptr()),
                                  Kp, ctypes.c_void_p(sc.data_ptr()), _stream_ptr(stream)))
    return q, sc


def mx_gemm(qa, sa, qb, sb, epilogue=GPT2_EPI_BIAS, bias=None, residual=None, stream=None):
    """C = A B^T (+ epilogue) on MX operands (gpt2_mx_gemm): qa [M, K], qb [N, K] uint8
    codes with scales [K / 128, rows, 4]; returns bf16 C [M, N] (and GELU(C) for
    GPT2_EPI_BIAS_GELU)."""
    import torch
    M, K = qa.shape
    N = qb.shape[0]
    ldc = (N + 7) // 8 * 8
    c = torch.empty(M, ldc, dtype=torch.bfloat16, device=qa.device)
    c2 = torch.empty_like(c) if epilogue == GPT2_EPI_BIAS_GELU else None
    if residual is not None:
        r = torch.zeros(M, ldc, dtype=torch.bfloat16, device=qa.device)
        r[:, :N] = residual
        residual = r
    ptr = (lambda t: None if t is None else ctypes.c_void_p(t.data_ptr()))
    _check(lib().gpt2_mx_gemm(ptr(qa), ptr(sa), qa.stride(0), ptr(qb), ptr(sb), qb.stride(0), ptr(c), ldc, M, N, K,
                              epilogue, ptr(bias), ptr(residual), ptr(c2), _stream_ptr(stream)))
    return (c[:, :N], c2[:, :N]) if c2 is not None else c[:, :N]
