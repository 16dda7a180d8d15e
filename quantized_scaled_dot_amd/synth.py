"""Seeded synthetic inputs for the quantized attention forward.

This module only draws random tensors; it holds none of the method's
arithmetic.  The oracle and the GPU path receive the same tensors from it.

Recipe (for every workload): ``numpy.random.default_rng(seed)`` (PCG64),
float32 standard normals drawn in the order Q, K, per-channel K bias, V,
then the V outlier channels; K gets a bias drawn per (b, h, channel) with the
stated variance and added to every token (channel outliers that smoothing
removes); optionally a fixed number of V channels per (b, h), chosen without
replacement, are multiplied by a factor; finally the tensors are rounded to
float16 / bfloat16 with round-to-nearest-even.  Q is [B, H, N, d]; K and V
are [B, Hkv, Nkv, d], which is Q's shape unless the workload sets grouped K/V
heads (Hkv < H) or a different key count (then the queries are the last N
positions of the Nkv-long sequence).  Shapes follow the workloads the method
is aimed at: LLM prefill (also with grouped K/V heads and with a query chunk
against a longer prefix), ViT, video DiT, long-context prefill, and decode
(one or four new queries per sequence against a long quantized cache).
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "float16" or "bfloat16"
    causal: bool
    blk_q: int
    blk_k: int
    bias_var: float
    sm_scale: float
    v_outlier_channels: int = 0
    v_outlier_scale: float = 1.0
    seed: int = 0
    Hkv_: int = 0         # K/V heads (0: H)
    Nkv_: int = 0         # keys (0: N)
    decode: bool = False  # N new queries against a quantized cache of Nkv keys (split over the keys)
    qk4: bool = False     # 4-bit QK^T (E2M1, a power-of-two scale per 32 channels) instead of INT8
    smooth_q: bool = False  # with qk4: Q smoothing (mean of each 32-query block, restored in INT8)
    pv4: bool = False     # with qk4: P~V in FP4 too (E2M1 P~ and V with E8M0 scales per 32 keys / tokens)
    q_bias_var: float = 0.0   # variance of a per-(b, h, channel) bias added to every query

    @property
    def Hkv(self):
        return self.Hkv_ or self.H

    @property
    def Nkv(self):
        return self.Nkv_ or self.N

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "float16" else torch.bfloat16

    @property
    def dtype_code(self):
        return 0 if self.dtype == "float16" else 1

    @property
    def ops(self):
        """Attention operation count 4*B*H*N*Nkv*d; causal: 4*B*H*d*(N*Nkv - N^2/2)
        (half of it when N = Nkv)."""
        pairs = self.N * self.Nkv - (self.N * self.N / 2 if self.causal else 0)
        return 4.0 * self.B * self.H * pairs * self.d

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _rsqrt32(x):
    return float(np.float32(1.0 / math.sqrt(x)))


WORKLOADS = {
    "tiny-f16-256": Workload("tiny-f16-256", 1, 2, 256, 64, "float16", False, 64, 64, 4.0, 0.125),
    "llm-prefill-4k-causal": Workload("llm-prefill-4k-causal", 4, 32, 4096, 128, "bfloat16", True, 128, 64,
                                      4.0, _rsqrt32(128)),
    "vit-2k-f16": Workload("vit-2k-f16", 16, 16, 2048, 64, "float16", False, 128, 64, 2.0, 0.125),
    "video-dit-32k": Workload("video-dit-32k", 1, 24, 32768, 128, "bfloat16", False, 128, 64, 4.0, _rsqrt32(128)),
    "long-prefill-128k-causal": Workload("long-prefill-128k-causal", 1, 8, 131072, 128, "bfloat16", True, 128, 64,
                                         4.0, _rsqrt32(128), v_outlier_channels=13, v_outlier_scale=8.0),
    # grouped K/V heads: 32 query heads on 8 K/V heads (4 queries per K/V head)
    "llm-prefill-8k-gqa-causal": Workload("llm-prefill-8k-gqa-causal", 1, 32, 8192, 128, "bfloat16", True, 128, 64,
                                          4.0, _rsqrt32(128), Hkv_=8),
    # a 4096-token query chunk at the end of a 32768-token prefix, grouped heads
    "chunked-prefill-4k-of-32k-gqa-causal": Workload("chunked-prefill-4k-of-32k-gqa-causal", 1, 32, 4096, 128,
                                                     "bfloat16", True, 128, 64, 4.0, _rsqrt32(128), Hkv_=8,
                                                     Nkv_=32768),
    # the video DiT shape with 4-bit QK^T
    "video-dit-32k-qk4": Workload("video-dit-32k-qk4", 1, 24, 32768, 128, "bfloat16", False, 128, 64, 4.0,
                                  _rsqrt32(128), qk4=True),
    # the same with P~V in FP4 as well: all matrix work on the FP4 instructions
    "video-dit-32k-fp4": Workload("video-dit-32k-fp4", 1, 24, 32768, 128, "bfloat16", False, 128, 64, 4.0,
                                  _rsqrt32(128), qk4=True, pv4=True),
    # the same with a channel bias in Q too (variance 4, like K's), 4-bit QK^T with Q smoothing
    "video-dit-32k-qk4-qsmooth": Workload("video-dit-32k-qk4-qsmooth", 1, 24, 32768, 128, "bfloat16", False, 128,
                                          64, 4.0, _rsqrt32(128), qk4=True, smooth_q=True, q_bias_var=4.0),
    # finer quantization granularity: a Q scale per 32 rows, a K scale per 16 keys
    "llm-prefill-4k-causal-fine": Workload("llm-prefill-4k-causal-fine", 4, 32, 4096, 128, "bfloat16", True, 32, 16,
                                           4.0, _rsqrt32(128)),
    # decode: one new query per sequence (32 query heads on 8 K/V heads) against a
    # 32768-token quantized cache, batch 16; and 4 speculative queries against 131072
    "decode-32k-gqa": Workload("decode-32k-gqa", 16, 32, 1, 128, "bfloat16", True, 128, 64, 4.0, _rsqrt32(128),
                               Hkv_=8, Nkv_=32768, decode=True),
    "decode-128k-gqa-4q": Workload("decode-128k-gqa-4q", 4, 32, 4, 128, "bfloat16", True, 128, 64, 4.0,
                                   _rsqrt32(128), Hkv_=8, Nkv_=131072, decode=True),
    # lengths that are not tile multiples: 3000 queries at the end of 3500 keys
    "llm-prefill-ragged-3000-of-3500-gqa-causal": Workload("llm-prefill-ragged-3000-of-3500-gqa-causal", 2, 32,
                                                           3000, 128, "bfloat16", True, 128, 64, 4.0,
                                                           _rsqrt32(128), Hkv_=8, Nkv_=3500),
}


def make_inputs(w: Workload, seed=None, device="cpu"):
    """Return Q [B, H, N, d] and K, V [B, Hkv, Nkv, d] as torch tensors of
    ``w.dtype`` on ``device``."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    kv_shape = (w.B, w.Hkv, w.Nkv, w.d)
    q = rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32)
    k = rng.standard_normal(kv_shape, dtype=np.float32)
    bias = rng.standard_normal((w.B, w.Hkv, 1, w.d), dtype=np.float32) * np.float32(math.sqrt(w.bias_var))
    k += bias
    v = rng.standard_normal(kv_shape, dtype=np.float32)
    if w.v_outlier_channels:
        for b in range(w.B):
            for h in range(w.Hkv):
                ch = rng.choice(w.d, size=w.v_outlier_channels, replace=False)
                v[b, h][:, ch] *= np.float32(w.v_outlier_scale)
    if w.q_bias_var:   # drawn last, so the other tensors keep their draws
        q += rng.standard_normal((w.B, w.H, 1, w.d), dtype=np.float32) * np.float32(math.sqrt(w.q_bias_var))
    out = []
    for a in (q, k, v):
        t = torch.from_numpy(a).to(w.torch_dtype)
        out.append(t.to(device) if device != "cpu" else t)
    return tuple(out)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a float16/bfloat16 CPU tensor as a uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
