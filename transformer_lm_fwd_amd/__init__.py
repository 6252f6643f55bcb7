"""MI355X-native GPT-2 training step: forward, backward and AdamW as hand-written
gfx950 HIP kernels behind the C ABI of include/gpt2.h, with a ctypes binding."""
from .binding import (Arena, Generator, Gpt2Error, sample_topk, GPT2_BF16, GPT2_FP32, arena_bytes, lib,  # noqa: F401
                      num_parameters)
