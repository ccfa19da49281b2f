"""Seeded synthetic inputs for the Grok-1 attention sub-layer core.

This module only draws numbers: it holds none of the method's arithmetic
(no RoPE, no norm, no attention, no projection). Both the fp64 oracle's tests
and the GPU path's tests and benchmark take their inputs from here, so the two
sides see exactly the same values.

Conventions
-----------
* Generator: ``numpy.random.Generator(PCG64(seed))``.
* Real-valued tensors are drawn as float32 ``standard_normal`` samples. A
  bf16 tensor is that float32 sample rounded to the nearest bf16
  (round-half-to-even) and is handed out as its raw ``uint16`` bit pattern.
* int8 weights are uniform integers in [-127, 127].
* Sequence lengths of the ragged decode workload are uniform integers in
  [512, 8192] (both ends included).

The five workloads mirror the shapes the pages describe for Grok-1
(48 query heads, 8 KV heads, head size 128, context 8192, model width 6144):
see ``WORKLOADS``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "Workload",
    "WORKLOADS",
    "rng",
    "normal_f32",
    "normal_bf16",
    "int8_uniform",
    "make_prefill_inputs",
    "make_decode_inputs",
    "make_sublayer_inputs",
    "make_decode_sublayer_inputs",
    "make_chunk_inputs",
    "make_moe_inputs",
    "make_workload",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bits.

    Encoding of drawn samples only; NaN is not expected from a normal draw.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def normal_bf16(g: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """bf16 bits of N(0,1) float32 draws; drawn in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(g.standard_normal(size=e - s, dtype=np.float32))
    return out.reshape(shape)


def int8_uniform(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(-127, 128, size=shape, dtype=np.int8)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode" | "sublayer" | "decode_sublayer" | "chunk" | "moe"
    seed: int
    dtype: str  # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int = 1  # query tokens per sequence
    Tmax: int = 0  # KV-cache capacity (decode)
    d_model: int = 0  # sub-layer width
    logit_scale_factor: float = 1.0  # multiplies 1/sqrt(D)
    softcap: float = 30.0
    rope_base: float = 10000.0
    eps: float = 1e-5
    d_ffn: int = 0       # MoE expert width
    n_experts: int = 0   # MoE
    top_k: int = 0       # MoE
    ragged: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def attn_mult(self) -> float:
        """Logit multiplier, returned as the float32 value passed to kernels."""
        return float(np.float32(self.logit_scale_factor / math.sqrt(self.D)))


WORKLOADS = {
    # Tiny fp32 causal prefill: one KV head shared by six query heads.
    "prefill_f32_t16": Workload(
        name="prefill_f32_t16", kind="prefill", seed=1001, dtype="f32",
        B=1, T=16, Hq=6, Hkv=1, D=32),
    # Single-token decode against a full 8192-slot cache.
    "decode_b1_t8192": Workload(
        name="decode_b1_t8192", kind="decode", seed=1002, dtype="bf16",
        B=1, Hq=48, Hkv=8, D=128, Tmax=8192),
    # 8k causal prefill with the logit multiplier raised 4x.
    "prefill_b1_t8192": Workload(
        name="prefill_b1_t8192", kind="prefill", seed=1003, dtype="bf16",
        B=1, T=8192, Hq=48, Hkv=8, D=128, logit_scale_factor=4.0),
    # 32 sequences of lengths uniform in [512, 8192], one new token each.
    "decode_ragged_b32_t8192": Workload(
        name="decode_ragged_b32_t8192", kind="decode", seed=1004, dtype="bf16",
        B=32, Hq=48, Hkv=8, D=128, Tmax=8192, ragged=True),
    # Full attention sub-layer: norm, int8 projections, RoPE, attention, norm.
    "sublayer_b4_t2048": Workload(
        name="sublayer_b4_t2048", kind="sublayer", seed=1005, dtype="bf16",
        B=4, T=2048, Hq=48, Hkv=8, D=128, d_model=6144),
    # Decode-time sub-layer: one new token against a full 8192-slot cache.
    "decode_sublayer_b1_t8192": Workload(
        name="decode_sublayer_b1_t8192", kind="decode_sublayer", seed=1006, dtype="bf16",
        B=1, Hq=48, Hkv=8, D=128, Tmax=8192, d_model=6144),
    # Decode-time sub-layer over 32 sequences of lengths uniform in [512, 8192].
    "decode_sublayer_b32_t8192": Workload(
        name="decode_sublayer_b32_t8192", kind="decode_sublayer", seed=1007, dtype="bf16",
        B=32, Hq=48, Hkv=8, D=128, Tmax=8192, d_model=6144, ragged=True),
    # Chunked prefill: 512 new tokens per sequence after a cached prefix of
    # uniform length in [0, 7680] (4 sequences).
    "prefill_chunk_b4_t512": Workload(
        name="prefill_chunk_b4_t512", kind="chunk", seed=1008, dtype="bf16",
        B=4, T=512, Hq=48, Hkv=8, D=128, Tmax=8192),
    # MoE FFN sub-layer: 4 x 2048 tokens, 8 experts 6144 -> 32768 -> 6144, top-2.
    "moe_b4_t2048": Workload(
        name="moe_b4_t2048", kind="moe", seed=1009, dtype="bf16",
        B=4, T=2048, Hq=0, Hkv=0, D=0, d_model=6144, d_ffn=32768, n_experts=8, top_k=2),
}


def make_prefill_inputs(B, T, Hq, Hkv, D, seed, dtype="bf16", key_pad_frac=0.0):
    """q [B,T,Hq,D], k/v [B,T,Hkv,D]; optional key-padding mask [B,T] (1 = keep).

    With ``key_pad_frac > 0`` each key is padding with that probability.
    """
    g = rng(seed)
    draw = normal_f32 if dtype == "f32" else normal_bf16
    q = draw(g, (B, T, Hq, D))
    k = draw(g, (B, T, Hkv, D))
    v = draw(g, (B, T, Hkv, D))
    key_valid = None
    if key_pad_frac > 0:
        key_valid = (g.random((B, T)) >= key_pad_frac).astype(np.uint8)
    return {"q": q, "k": k, "v": v, "key_valid": key_valid}


def make_decode_inputs(B, Hq, Hkv, D, Tmax, seed, lengths=None, ragged=False):
    """Cache [B,Tmax,Hkv,D] (every slot finite N(0,1), valid or not), new q/k/v
    [B,1,H,D], and per-sequence step = length-1 (the new token's slot).

    ``lengths[b]`` counts the new token, so the attended keys are
    slots ``[0, lengths[b])`` after the append.
    """
    g = rng(seed)
    k_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    v_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    q = normal_bf16(g, (B, 1, Hq, D))
    k_new = normal_bf16(g, (B, 1, Hkv, D))
    v_new = normal_bf16(g, (B, 1, Hkv, D))
    if lengths is None:
        if ragged:
            lengths = g.integers(512, Tmax + 1, size=B)
        else:
            lengths = np.full(B, Tmax)
    lengths = np.asarray(lengths, dtype=np.int32)
    step = (lengths - 1).astype(np.int32)
    return {"k_cache": k_cache, "v_cache": v_cache, "q": q, "k_new": k_new,
            "v_new": v_new, "step": step, "kv_len": lengths.copy()}


def make_sublayer_inputs(B, T, d_model, Hq, Hkv, D, seed, scale=0.02 / 127,
                         distinct_scales=False):
    """x [B,T,d] bf16; int8 weights Wq [d,Hq*D], Wk/Wv [d,Hkv*D], Wo [Hq*D,d];
    per-output-channel float32 scales (constant ``scale``, or drawn per channel)."""
    g = rng(seed)
    x = normal_bf16(g, (B, T, d_model))
    wq = int8_uniform(g, (d_model, Hq * D))
    wk = int8_uniform(g, (d_model, Hkv * D))
    wv = int8_uniform(g, (d_model, Hkv * D))
    wo = int8_uniform(g, (Hq * D, d_model))

    def sc(n):
        if distinct_scales:
            return (scale * g.uniform(0.5, 1.5, size=n)).astype(np.float32)
        return np.full(n, scale, dtype=np.float32)

    return {"x": x, "wq": wq, "wk": wk, "wv": wv, "wo": wo,
            "sq": sc(Hq * D), "sk": sc(Hkv * D), "sv": sc(Hkv * D), "so": sc(d_model)}


def make_decode_sublayer_inputs(B, d_model, Hq, Hkv, D, Tmax, seed, lengths=None, ragged=False,
                                scale=0.02 / 127, distinct_scales=False):
    """One new token per sequence: x [B,1,d] bf16, the int8 weights and scales
    of ``make_sublayer_inputs``, and a cache [B,Tmax,Hkv,D] (every slot finite
    N(0,1)) with step = length-1 (the new token's slot)."""
    g = rng(seed)
    k_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    v_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    if lengths is None:
        lengths = g.integers(512, Tmax + 1, size=B) if ragged else np.full(B, Tmax)
    lengths = np.asarray(lengths, dtype=np.int32)
    out = make_sublayer_inputs(B, 1, d_model, Hq, Hkv, D, int(g.integers(1 << 31)), scale,
                               distinct_scales)
    out.update({"k_cache": k_cache, "v_cache": v_cache, "step": (lengths - 1).astype(np.int32),
                "kv_len": lengths.copy()})
    return out


def make_chunk_inputs(B, T, Hq, Hkv, D, Tmax, seed, offsets=None):
    """A cache [B,Tmax,Hkv,D] (every slot finite N(0,1); slots below the offset
    are the cached prefix, used as already rotated), T new q/k/v rows per
    sequence, and step = offset = the cached length, uniform in [0, Tmax-T]."""
    g = rng(seed)
    k_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    v_cache = normal_bf16(g, (B, Tmax, Hkv, D))
    q = normal_bf16(g, (B, T, Hq, D))
    k_new = normal_bf16(g, (B, T, Hkv, D))
    v_new = normal_bf16(g, (B, T, Hkv, D))
    if offsets is None:
        offsets = g.integers(0, Tmax - T + 1, size=B)
    step = np.asarray(offsets, dtype=np.int32)
    return {"k_cache": k_cache, "v_cache": v_cache, "q": q, "k_new": k_new, "v_new": v_new,
            "step": step}


def make_moe_inputs(B, T, d_model, d_ffn, n_experts, seed, scale_up=0.02 / 127, scale_down=0.02 / 127,
                    router_std=None, distinct_scales=False):
    """x [B,T,d] bf16; router weights [d, E] float32 N(0, router_std^2)
    (default 1.5/sqrt(d): logits of standard deviation 1.5 for unit-RMS rows);
    per expert the int8 weights Wg, Wv [d, F] and W1 [F, d] (uniform in
    [-127, 127]) with float32 per-channel scales."""
    g = rng(seed)
    x = normal_bf16(g, (B, T, d_model))
    std = router_std if router_std is not None else 1.5 / math.sqrt(d_model)
    w_router = (normal_f32(g, (d_model, n_experts)) * np.float32(std)).astype(np.float32)

    def sc(n, s):
        if distinct_scales:
            return (s * g.uniform(0.5, 1.5, size=n)).astype(np.float32)
        return np.full(n, s, dtype=np.float32)

    experts = []
    for _ in range(n_experts):
        wg = int8_uniform(g, (d_model, d_ffn))
        wv = int8_uniform(g, (d_model, d_ffn))
        w1 = int8_uniform(g, (d_ffn, d_model))
        experts.append((wg, sc(d_ffn, scale_up), wv, sc(d_ffn, scale_up), w1, sc(d_model, scale_down)))
    return {"x": x, "w_router": w_router, "experts": experts}


def make_workload(name: str) -> dict:
    """All inputs of one named workload at its full size."""
    w = WORKLOADS[name]
    if w.kind == "prefill":
        return make_prefill_inputs(w.B, w.T, w.Hq, w.Hkv, w.D, w.seed, w.dtype)
    if w.kind == "decode":
        return make_decode_inputs(w.B, w.Hq, w.Hkv, w.D, w.Tmax, w.seed, ragged=w.ragged)
    if w.kind == "moe":
        return make_moe_inputs(w.B, w.T, w.d_model, w.d_ffn, w.n_experts, w.seed)
    if w.kind == "chunk":
        return make_chunk_inputs(w.B, w.T, w.Hq, w.Hkv, w.D, w.Tmax, w.seed)
    if w.kind == "decode_sublayer":
        return make_decode_sublayer_inputs(w.B, w.d_model, w.Hq, w.Hkv, w.D, w.Tmax, w.seed,
                                           ragged=w.ragged)
    return make_sublayer_inputs(w.B, w.T, w.d_model, w.Hq, w.Hkv, w.D, w.seed)
