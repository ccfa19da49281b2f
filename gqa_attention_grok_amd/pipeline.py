"""The hot path as sequences of C-ABI calls on preallocated device buffers.

Nothing here computes: each step only orders calls into ``libgrokattn.so`` on
the current stream, with every output buffer allocated once up front (torch
owns device memory).

* ``DecodeStep``   -- one decoded token per sequence (Grok-1 walkthrough, ch. 4
  "model.py close reading, part 1", §4.4): RoPE q and the new k at step[b],
  append k/v to the cache, attend slots [0, step[b]+1) -- one fused call.
* ``PrefillStep``  -- a prompt with no cache (same page, §4.3.1 and §4.5):
  RoPE q and k at positions 0..T-1, causal GQA attention (optionally with q
  rotated inside the attention kernel).
* ``SublayerStep`` -- the attention half of a decoder layer (ch. 6 "model.py
  close reading, part 3", §6.3.1): h = x + norm(Wo . attn(rope(Wq n),
  rope(Wk n), Wv n)) with n = norm(x).
* ``ChunkStep``    -- a chunk of T new tokens per sequence after a cached
  prefix (ch. 4 §4.4, ch. 6 §6.6.1): RoPE q and k at step[b] + t, append k/v,
  causal attention on absolute positions over the cache.
* ``DecodeSublayerStep`` -- the same sub-layer for one new token per sequence
  against the KV memory (ch. 4 §4.4, ch. 6 §6.6): the projections are few-row
  products that stream the int8 weights once, and the attention is the
  one-token decode over slots [0, step[b]+1).
* ``MoeStep``      -- the FFN half of a decoder layer (ch. 6 §6.2, §6.3.1;
  ch. 3 "Configuration and hyperparameters" §3.5; ch. 2 "Overall
  architecture" §2.2): y = x + norm(sum of the two routed GeGLU experts'
  outputs, weighted by their router probabilities) -- one call.
"""
from __future__ import annotations

import torch

from . import (grok_attn_decode, grok_attn_decode_append, grok_attn_decode_workspace_bytes,
               grok_attn_prefill, grok_attn_prefill_chunk, grok_attn_prefill_rope,
               grok_attn_prefill_rope_workspace_bytes,
               grok_decode_out, grok_decode_out_workspace_bytes, grok_decode_qkv, grok_kv_append, grok_linear_int8, grok_linear_int8_gemv,
               grok_linear_int8_pack, grok_moe_ffn, grok_moe_interleave, grok_moe_workspace_bytes,
               grok_prefill_qkv, grok_prefill_qkv_workspace_bytes, grok_rmsnorm, grok_rope)


def capture(step) -> "torch.cuda.CUDAGraph":
    """Record one call of ``step`` into a HIP graph (torch's CUDAGraph API on
    ROCm) so that it can be replayed without host launch overhead. The step's
    kernels are launched on torch's current stream, which is the capture stream
    inside the context; none of them records a memset."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


class DecodeStep:
    """One decoded token per sequence: RoPE q and the new k at step[b], append
    k/v at slot step[b], attend slots [0, step[b]+1). Fused (default): one call
    (split kernel with the append, then the combine), q left as given;
    unfused: the append call (rotating q in place), then the decode call."""

    def __init__(self, k_cache, v_cache, q, k_new, v_new, step, attn_mult, softcap=30.0,
                 rope_base=10000.0, fused=True):
        self.k_cache, self.v_cache = k_cache, v_cache
        self.q, self.k_new, self.v_new, self.step = q, k_new, v_new, step
        self.attn_mult, self.softcap, self.rope_base = attn_mult, softcap, rope_base
        self.fused = fused
        B, Tmax, Hkv, D = k_cache.shape
        Hq = q.shape[2]
        dev = q.device
        self.out = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device=dev)
        self.kv_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        nbytes = grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D)
        self.workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def attend(self):
        """The attention launches alone (cache already holding the new token)."""
        grok_attn_decode(self.q, self.k_cache, self.v_cache, self.kv_len, self.out,
                         self.workspace, self.attn_mult, self.softcap, status=self.status)

    def __call__(self):
        if self.fused:
            grok_attn_decode_append(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                                    self.step, self.out, self.workspace, self.attn_mult,
                                    self.softcap, new_step=self.kv_len, status=self.status,
                                    rope_base=self.rope_base)
        else:
            grok_kv_append(self.k_cache, self.v_cache, self.k_new, self.v_new, self.step,
                           q_inout=self.q, new_step=self.kv_len, status=self.status,
                           rope_base=self.rope_base)
            self.attend()
        return self.out


class PrefillStep:
    """A prompt with no cache: RoPE of q and k at positions 0..T-1, then the
    causal attention. fused_rope (bf16, D = 128): k is rotated in place by its
    own pass and q inside the attention kernel (q is left unrotated);
    otherwise (the default) both are rotated in place first."""

    def __init__(self, q, k, v, attn_mult, softcap=30.0, rope_base=10000.0, key_valid=None, fused_rope=False):
        self.q, self.k, self.v = q, k, v
        self.attn_mult, self.softcap, self.rope_base = attn_mult, softcap, rope_base
        self.key_valid = key_valid
        B, T, Hq, D = q.shape
        self.fused_rope = fused_rope
        self.out = torch.empty((B, T, Hq * D), dtype=q.dtype, device=q.device)
        self.ws = (torch.empty(grok_attn_prefill_rope_workspace_bytes(T, D), dtype=torch.uint8, device=q.device)
                   if fused_rope else None)

    def rope(self):
        if not self.fused_rope:
            grok_rope(self.q, None, self.rope_base)
        grok_rope(self.k, None, self.rope_base)

    def attend(self):
        if self.fused_rope:
            return grok_attn_prefill_rope(self.q, self.k, self.v, self.out, self.ws, self.attn_mult, self.softcap,
                                          key_valid=self.key_valid, rope_base=self.rope_base)
        return grok_attn_prefill(self.q, self.k, self.v, self.out, self.attn_mult, self.softcap,
                                 key_valid=self.key_valid)

    def __call__(self):
        self.rope()
        return self.attend()


class ChunkStep:
    """Chunked prefill: append (RoPE q in place and k into the cache at
    step[b] + t), then the chunk's attention over cache slots [0, step[b] + t]."""

    def __init__(self, k_cache, v_cache, q, k_new, v_new, step, attn_mult, softcap=30.0,
                 rope_base=10000.0):
        self.k_cache, self.v_cache = k_cache, v_cache
        self.q, self.k_new, self.v_new, self.step = q, k_new, v_new, step
        self.attn_mult, self.softcap, self.rope_base = attn_mult, softcap, rope_base
        B, T, Hq, D = q.shape
        dev = q.device
        self.out = torch.empty((B, T, Hq * D), dtype=torch.bfloat16, device=dev)
        self.new_step = torch.empty_like(step)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)

    def append(self):
        grok_kv_append(self.k_cache, self.v_cache, self.k_new, self.v_new, self.step,
                       q_inout=self.q, new_step=self.new_step, status=self.status,
                       rope_base=self.rope_base)

    def attend(self):
        return grok_attn_prefill_chunk(self.q, self.k_cache, self.v_cache, self.step, self.out,
                                       self.attn_mult, self.softcap, status=self.status)

    def __call__(self):
        self.append()
        return self.attend()


class SublayerStep:
    """Attention sub-layer with unit-scale norms and int8 projections.
    fused=True runs the Q/K/V projections, RoPE of q and k and the writes of
    q, k, v as one launch (grok_prefill_qkv); fused=False runs three
    projections and two RoPE passes."""

    def __init__(self, x, wq, sq, wk, sk, wv, sv, wo, so, Hq, Hkv, D, attn_mult, softcap=30.0,
                 eps=1e-5, rope_base=10000.0, key_valid=None, fused=True):
        self.fused = fused
        self.x = x
        self.w = (wq, sq, wk, sk, wv, sv, wo, so)
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.attn_mult, self.softcap, self.eps, self.rope_base = attn_mult, softcap, eps, rope_base
        self.key_valid = key_valid
        B, T, d = x.shape
        dev = x.device
        bf = torch.bfloat16
        self.n = torch.empty((B, T, d), dtype=bf, device=dev)
        self.q = torch.empty((B, T, Hq, D), dtype=bf, device=dev)
        self.k = torch.empty((B, T, Hkv, D), dtype=bf, device=dev)
        self.v = torch.empty((B, T, Hkv, D), dtype=bf, device=dev)
        self.attn = torch.empty((B, T, Hq * D), dtype=bf, device=dev)
        self.o = torch.empty((B, T, d), dtype=bf, device=dev)
        self.y = torch.empty((B, T, d), dtype=bf, device=dev)
        self.ws = torch.empty(grok_prefill_qkv_workspace_bytes(T, D), dtype=torch.uint8, device=dev)

    def __call__(self):
        wq, sq, wk, sk, wv, sv, wo, so = self.w
        grok_rmsnorm(self.x, self.n, eps=self.eps)
        if self.fused:
            grok_prefill_qkv(self.n, wq, sq, wk, sk, wv, sv, self.q, self.k, self.v, self.ws,
                             rope_base=self.rope_base)
        else:
            grok_linear_int8(self.n, wq, sq, self.q)
            grok_linear_int8(self.n, wk, sk, self.k)
            grok_linear_int8(self.n, wv, sv, self.v)
            grok_rope(self.q, None, self.rope_base)
            grok_rope(self.k, None, self.rope_base)
        grok_attn_prefill(self.q, self.k, self.v, self.attn, self.attn_mult, self.softcap,
                          key_valid=self.key_valid)
        grok_linear_int8(self.attn, wo, so, self.o)
        grok_rmsnorm(self.o, self.y, residual=self.x, eps=self.eps)
        return self.y


class DecodeSublayerStep:
    """Attention sub-layer for one new token per sequence, with KV memory:
    n = norm(x); q, k, v = n . W (one launch for the three); RoPE q and k at
    step[b] and append k, v at slot step[b]; decode attention over slots
    [0, step[b]+1); y = x + norm(attn . Wo) (one launch with fused=True). x
    [B, 1, d]; the caches are
    updated in place, the step counter is not advanced (kv_len = step + 1).
    The int8 weights are repacked once, here, into the layout the few-row
    product streams."""

    def __init__(self, x, k_cache, v_cache, step, wq, sq, wk, sk, wv, sv, wo, so, Hq, Hkv, D,
                 attn_mult, softcap=30.0, eps=1e-5, rope_base=10000.0, fused=True, fused_back=None):
        self.x, self.k_cache, self.v_cache, self.step = x, k_cache, v_cache, step
        self.fused = fused
        self.fused_back = fused if fused_back is None else fused_back
        # the fused pre-norm keeps x on chip: up to 4 rows of up to 8192 values in all
        self.max_prenorm_rows = min(4, 32768 // x.shape[-1])
        self.w_args = (wq, sq, wk, sk, wv, sv, wo, so)
        self.Hq, self.Hkv, self.D = Hq, Hkv, D
        self.packed = tuple(grok_linear_int8_pack(w_) for w_ in (wq, wk, wv, wo))
        self.scales = (sq, sk, sv, so)
        self.attn_mult, self.softcap, self.eps, self.rope_base = attn_mult, softcap, eps, rope_base
        B, _, d = x.shape
        Tmax = k_cache.shape[1]
        dev = x.device
        bf = torch.bfloat16
        self.n = torch.empty((B, 1, d), dtype=bf, device=dev)
        self.q = torch.empty((B, 1, Hq, D), dtype=bf, device=dev)
        self.k = torch.empty((B, 1, Hkv, D), dtype=bf, device=dev)
        self.v = torch.empty((B, 1, Hkv, D), dtype=bf, device=dev)
        self.attn = torch.empty((B, 1, Hq * D), dtype=bf, device=dev)
        self.o = torch.empty((B, 1, d), dtype=bf, device=dev)
        self.y = torch.empty((B, 1, d), dtype=bf, device=dev)
        self.kv_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        nbytes = grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D)
        self.attn_ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
        # zeroed once: the back half's arrival counter is left at zero by every call
        self.out_ws = torch.zeros(grok_decode_out_workspace_bytes(B, Hq * D, d), dtype=torch.uint8, device=dev)

    def project_qkv(self):
        pq, pk, pv, _ = self.packed
        sq, sk, sv, _ = self.scales
        grok_linear_int8_gemv(self.n, [pq, pk, pv], [sq, sk, sv], [self.q, self.k, self.v])

    def project_out(self):
        grok_linear_int8_gemv(self.attn, [self.packed[3]], [self.scales[3]], [self.o])

    def back(self):
        """output projection -> post-norm -> + x. Fused: one launch (for up to
        4 rows; two inside the call for more); unfused: projection, norm."""
        if self.fused_back:
            grok_decode_out(self.attn, self.packed[3], self.scales[3], self.x, self.y, self.out_ws, eps=self.eps)
        else:
            self.project_out()
            grok_rmsnorm(self.o, self.y, residual=self.x, eps=self.eps)

    def front(self):
        """norm -> Q|K|V -> RoPE -> cache slot. Fused into one launch (the norm
        too when the rows fit on chip); unfused: norm, projection, append."""
        pq, pk, pv, _ = self.packed
        sq, sk, sv, _ = self.scales
        if self.fused:
            B = self.x.shape[0]
            prenorm = B <= self.max_prenorm_rows
            if not prenorm:
                grok_rmsnorm(self.x, self.n, eps=self.eps)
            grok_decode_qkv(self.x if prenorm else self.n, pq, sq, pk, sk, pv, sv, self.q, self.k_cache,
                            self.v_cache, self.step, new_step=self.kv_len, status=self.status,
                            prenorm=prenorm, eps=self.eps, rope_base=self.rope_base)
        else:
            grok_rmsnorm(self.x, self.n, eps=self.eps)
            self.project_qkv()
            grok_kv_append(self.k_cache, self.v_cache, self.k, self.v, self.step, q_inout=self.q,
                           new_step=self.kv_len, status=self.status, rope_base=self.rope_base)

    def __call__(self):
        self.front()
        grok_attn_decode(self.q, self.k_cache, self.v_cache, self.kv_len, self.attn, self.attn_ws,
                         self.attn_mult, self.softcap, status=self.status)
        self.back()
        return self.y


class MoeStep:
    """MoE FFN sub-layer: the experts' gate and value weights are interleaved
    once at construction; each call is one grok_moe_ffn on preallocated
    buffers. `experts` is a list of (wg, sg, wv, sv, w1, s1) device tensors."""

    def __init__(self, x, w_router, experts, k=2, eps=1e-5):
        self.x, self.w_router, self.k, self.eps = x, w_router, k, eps
        d, E = w_router.shape
        T = x.numel() // d
        F = experts[0][4].shape[0]
        dev = x.device
        self.wgv, self.sgv, self.w1, self.s1 = [], [], [], []
        for wg, sg, wv, sv, w1, s1 in experts:
            a, b = grok_moe_interleave(wg, sg, wv, sv)
            self.wgv.append(a)
            self.sgv.append(b)
            self.w1.append(w1)
            self.s1.append(s1)
        self.ws = torch.empty(grok_moe_workspace_bytes(T, d, F, E, k), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(x)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.gates = torch.empty((T, k), dtype=torch.float32, device=dev)

    def __call__(self):
        return grok_moe_ffn(self.x, self.w_router, self.wgv, self.sgv, self.w1, self.s1, self.out, self.ws,
                            k=self.k, eps=self.eps, idx=self.idx, gates=self.gates)
