"""Plain float64 reference for Grok-1's attention sub-layer core (test infrastructure).

Sources (the Grok-1 walkthrough pages; section numbers are the pages' own):

* [ch4] "model.py close reading, part 1: RMSNorm, RoPE, GQA Attention"
  (yingwang.github.io/grok-1/04-model-1/): §4.1 int8 ``Linear``, §4.2 RMSNorm,
  §4.3 ``rotate_half``, §4.3.1 ``RotaryEmbedding`` (rotation-matrix form),
  §4.3.1.1 NeoX vs interleaved pairing, §4.4 RoPE-before-cache and the memory
  mask, §4.4.1 the 6x6 causal mask figure, §4.5.2 GQA logits and softcap,
  §4.5.3 mask fill and fp32 softmax, §4.5.4 P.V and head merge.
* [ch6] "model.py close reading, part 3: block assembly and sharding"
  (yingwang.github.io/grok-1/06-model-3/): §6.3/§6.3.1 sandwich norm,
  §6.4.2 causal x padding mask, §6.6 KV memory.
* [ch3] "Configuration and hyperparameters" (yingwang.github.io/grok-1/03-config/):
  §3.3 / §3.3.2 attention constants, §3.5 the router.
* [ch2] "Overall architecture" (yingwang.github.io/grok-1/02-architecture/):
  §2.2 data flow of a layer, §2.5.1 unnormalised top-2 gates.
* [ch6] §6.2 the gated FFN of one expert (``jax.nn.gelu`` on the gate).

Everything is float64 unless a step's precision is fixed by the pages (the
RoPE phase is float32 there, [ch4] §4.3.1). Results are rounded to the output
dtype only where an exported operation hands back a tensor (``out=`` below),
which is where the pages' code casts back to the forward dtype.

Readings where the pages are silent:

* RoPE ``inv_freq[i]`` is the float32 nearest to ``base**(-2i/D)``; the phase
  ``t*inv_freq`` is one float32 product ([ch4] §4.3.1); cos/sin in float64.
* The logit multiplier is applied before the softcap, the softcap before the
  mask fill, and masked logits are ``-1e30`` ([ch4] §4.5.2, §4.5.3). A row
  with no valid key therefore becomes a uniform average over every key.
* The softmax probabilities and logits stay float64 (parity unpinned: the
  pages do not fix whether the reference rounds them to bf16).
* ``kv_append`` raises when ``step + T`` exceeds the cache (the pages do not
  say what happens then).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "NEG_FILL",
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "round_bf16",
    "round_f32",
    "round_to",
    "softcap",
    "rmsnorm",
    "linear_int8",
    "rotate_half",
    "rope_inv_freq",
    "rope",
    "kv_append",
    "attention_mask",
    "softmax",
    "attention",
    "attention_rows",
    "decode_step",
    "sublayer",
    "decode_sublayer",
    "chunk_prefill",
    "gelu",
    "moe_route",
    "expert_ffn",
    "moe_sublayer",
    "kv_cache_bytes",
]

# [ch4] §4.5.3: masked logits are replaced by -1e30 (not -inf).
NEG_FILL = -1e30


# --------------------------------------------------------------------------
# dtype helpers (bf16 is handled as raw uint16 bit patterns)
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits; below 2**-126 the spacing is fixed at
    2**-133 (bf16 subnormals); beyond the largest finite bf16 the result is inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if np.any(fin):
        xf = x[fin]
        _, e = np.frexp(xf)  # xf = m * 2**e, 0.5 <= |m| < 1
        q = np.maximum(e - 8, -133).astype(np.float64)
        step = np.ldexp(1.0, q.astype(np.int64))
        r = np.rint(xf / step) * step  # rint: ties to even
        max_bf16 = float(np.ldexp(255.0 / 128.0, 127))  # (2 - 2**-7) * 2**127
        r = np.where(np.abs(r) > max_bf16, np.sign(r) * np.inf, r)
        out[fin] = r
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """Bits of ``round_bf16(x)`` (the value is exact in float32, so the cast is exact)."""
    r = round_bf16(x).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, out):
    if out is None:
        return np.asarray(x, dtype=np.float64)
    if out == "bf16":
        return round_bf16(x)
    if out == "f32":
        return round_f32(x)
    raise ValueError(f"unknown output dtype {out!r}")


# --------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------
def softcap(z, cap=30.0):
    """[ch4] §4.5.2 / [ch3] §3.3.2: logits are soft-capped as cap*tanh(z/cap)."""
    return cap * np.tanh(np.asarray(z, dtype=np.float64) / cap)


def rmsnorm(x, gamma=None, eps=1e-5, residual=None, out=None):
    """[ch4] §4.2: y = gamma * x / sqrt(mean(x^2) + eps) over the last axis.

    No mean subtraction and no bias. ``gamma=None`` is the unit scale.
    ``residual`` (optional) is added afterwards, as the sandwich norm does
    ([ch6] §6.3.1: h += norm(attn)); the normalised value is first handed
    back in the output dtype, then added and rounded again.
    """
    x = np.asarray(x, dtype=np.float64)
    mean_sq = np.mean(np.square(x), axis=-1, keepdims=True)
    y = x / np.sqrt(mean_sq + eps)
    if gamma is not None:
        y = np.asarray(gamma, dtype=np.float64) * y
    y = round_to(y, out)
    if residual is not None:
        y = round_to(np.asarray(residual, dtype=np.float64) + y, out)
    return y


def linear_int8(x, w_int8, scales, out=None):
    """[ch4] §4.1: y = x @ (w * s), w int8 [in, out], s float32 [out].

    The dequantised weight is ``w[k, n] * s[n]`` (one scale per output
    channel, broadcast along the input axis) and is kept exact in float64.
    Leading axes of ``x`` are flattened and restored.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_int8, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    lead = x.shape[:-1]
    y = x.reshape(-1, x.shape[-1]) @ (w * s[None, :])
    return round_to(y.reshape(*lead, w.shape[1]), out)


def rotate_half(x):
    """[ch4] §4.3: split the last axis into halves (x1, x2) -> (-x2, x1)."""
    half = x.shape[-1] // 2
    return np.concatenate((-x[..., half:], x[..., :half]), axis=-1)


def rope_inv_freq(D, base=10000.0) -> np.ndarray:
    """[ch4] §4.3.1: one frequency per pair i < D/2, base**(-2i/D), as float32."""
    if D % 2:
        raise ValueError("RoPE needs an even head size")
    i2 = np.arange(0, D, 2, dtype=np.float64)
    return np.asarray(np.power(float(base), -i2 / D), dtype=np.float32)


def rope(x, positions, base=10000.0, out=None):
    """[ch4] §4.3.1: x' = x*cos(phase) + rotate_half(x)*sin(phase).

    ``x`` is [B, T, H, D]; ``positions`` is [B, T] (offset + t). The phase is
    the float32 product position * inv_freq, tiled over both halves of the
    head so that element i pairs with i + D/2 (GPT-NeoX layout, §4.3.1.1).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    inv = rope_inv_freq(D, base)
    t = np.asarray(positions).astype(np.float32)
    phase = (t[..., None] * inv).astype(np.float32)  # [B, T, D/2], float32 product
    phase = np.concatenate((phase, phase), axis=-1)[:, :, None, :].astype(np.float64)
    y = x * np.cos(phase) + rotate_half(x) * np.sin(phase)
    return round_to(y, out)


def kv_append(k_cache, v_cache, k_new, v_new, step):
    """[ch4] §4.4: write new K/V rows at slot step[b] of each sequence's cache.

    Caches are [B, Tmax, Hkv, D]; new rows are [B, T, Hkv, D]; any dtype (the
    copy is bit-for-bit). Returns (k_cache', v_cache', new_step) with
    new_step = step + T; nothing else in the caches changes.
    """
    step = np.asarray(step, dtype=np.int64)
    B, Tmax = k_cache.shape[:2]
    T = k_new.shape[1]
    if np.any(step < 0) or np.any(step + T > Tmax):
        raise ValueError("cache write out of range")
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for b in range(B):
        s = int(step[b])
        kc[b, s:s + T] = k_new[b]
        vc[b, s:s + T] = v_new[b]
    return kc, vc, (step + T).astype(np.int32)


def attention_mask(q_pos, Tk, key_valid=None, kv_len=None) -> np.ndarray:
    """Boolean [B, Tq, Tk] mask: causal x padding x memory.

    [ch6] §6.4.2: mask[i, j] = 1[token_j is not pad] * 1[j <= i]; [ch4] §4.4:
    the memory mask keeps cache slots j < step + T. ``q_pos`` [B, Tq] holds each
    query's absolute position.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    j = np.arange(Tk, dtype=np.int64)
    m = j[None, None, :] <= q_pos[:, :, None]
    if key_valid is not None:
        m = m & (np.asarray(key_valid)[:, None, :] != 0)
    if kv_len is not None:
        m = m & (j[None, None, :] < np.asarray(kv_len, dtype=np.int64)[:, None, None])
    return m


def softmax(z, axis=-1):
    """Max-subtracted softmax ([ch4] §4.5.3)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q, k, v, mask, mult, cap=30.0, out=None, return_weights=False):
    """[ch4] §4.5.2-§4.5.4: grouped-query attention with softcap.

    q [B, Tq, Hq, D]; k, v [B, Tk, Hkv, D]; mask [B, Tq, Tk] (True = attend).
    Query head h uses KV head h // (Hq/Hkv): q is viewed as [B, Tq, Hkv, G, D]
    and K/V broadcast over G. Steps: logits = q.k in float64; *= mult;
    softcap; where(mask, logits, -1e30); softmax; weights . v; heads merged
    as [B, Tq, Hq*D] with head h in columns h*D .. h*D+D-1.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Tq, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    qg = q.reshape(B, Tq, Hkv, G, D)
    logits = np.einsum("bthHd,bThd->bhHtT", qg, k)
    logits = logits * mult
    logits = softcap(logits, cap)
    logits = np.where(np.asarray(mask, dtype=bool)[:, None, None, :, :], logits, NEG_FILL)
    w = softmax(logits, axis=-1)
    o = np.einsum("bhHtT,bThd->bthHd", w, v).reshape(B, Tq, Hq * D)
    o = round_to(o, out)
    if return_weights:
        return o, w
    return o


def attention_rows(q, k, v, b, t, h, mask_row, mult, cap=30.0):
    """One output row of ``attention``: query (b, t, h) against all keys of b.

    Same definition, evaluated for a single (sequence, position, head) so that
    sampled outputs of very large problems can be checked one by one.
    Returns the float64 [D] output of head h.
    """
    Hq, Hkv = q.shape[2], k.shape[2]
    g = h // (Hq // Hkv)
    qq = np.asarray(q[b, t, h], dtype=np.float64)
    kk = np.asarray(k[b, :, g], dtype=np.float64)
    vv = np.asarray(v[b, :, g], dtype=np.float64)
    z = softcap((kk @ qq) * mult, cap)
    z = np.where(np.asarray(mask_row, dtype=bool), z, NEG_FILL)
    return softmax(z) @ vv


def decode_step(k_cache, v_cache, q, k_new, v_new, step, mult, cap=30.0,
                base=10000.0, io="bf16"):
    """One decode step of one layer ([ch4] §4.4, §4.5).

    RoPE q and the new k at position step[b]; write k, v at slot step[b];
    attend slots [0, step[b] + 1) (memory mask; the causal mask of a single
    query is all-ones). Inputs are float64 values (already in the I/O dtype).
    Returns (out [B, 1, Hq*D], k_cache', v_cache', new_step).
    """
    B = q.shape[0]
    pos = np.asarray(step, dtype=np.int64).reshape(B, 1)
    qr = rope(q, pos, base, out=io)
    kr = rope(k_new, pos, base, out=io)
    kc, vc, new_step = kv_append(k_cache, v_cache, kr, np.asarray(v_new, np.float64), step)
    Tmax = kc.shape[1]
    mask = attention_mask(pos, Tmax, kv_len=new_step)
    o = attention(qr, kc, vc, mask, mult, cap, out=io)
    return o, kc, vc, new_step


def sublayer(x, wq, sq, wk, sk, wv, sv, wo, so, Hq, Hkv, D, mult, cap=30.0,
             eps=1e-5, base=10000.0, key_valid=None, io="bf16"):
    """Attention half of a decoder layer with no KV memory ([ch6] §6.3.1).

    h = x + norm(MHA(norm(x))) with unit-scale norms; MHA = int8 Q/K/V
    projections (no bias, [ch4] §4.5.1), RoPE at offset 0, causal (x padding)
    GQA attention, int8 output projection ([ch4] §4.5.4). Each step's result is
    handed on in the I/O dtype.
    """
    B, T, _ = x.shape
    n = rmsnorm(x, None, eps, out=io)
    q = linear_int8(n, wq, sq, out=io).reshape(B, T, Hq, D)
    k = linear_int8(n, wk, sk, out=io).reshape(B, T, Hkv, D)
    v = linear_int8(n, wv, sv, out=io).reshape(B, T, Hkv, D)
    pos = np.broadcast_to(np.arange(T), (B, T))
    q = rope(q, pos, base, out=io)
    k = rope(k, pos, base, out=io)
    mask = attention_mask(pos, T, key_valid=key_valid)
    a = attention(q, k, v, mask, mult, cap, out=io)
    o = linear_int8(a, wo, so, out=io)
    return rmsnorm(o, None, eps, residual=x, out=io)


def decode_sublayer(x, k_cache, v_cache, step, wq, sq, wk, sk, wv, sv, wo, so, Hq, Hkv, D, mult,
                    cap=30.0, eps=1e-5, base=10000.0, io="bf16"):
    """Attention half of a decoder layer for one new token per sequence, with
    KV memory ([ch6] §6.3.1 sandwich norm around [ch4] §4.5 attention; the
    memory update of [ch4] §4.4 and [ch6] §6.6).

    x [B, 1, d]; caches [B, Tmax, Hkv, D]; step [B] (the new token's slot and
    position). n = norm(x); q, k, v = int8 projections of n; q and k roped at
    step[b], k and v written to slot step[b]; attention over slots
    [0, step[b] + 1); y = x + norm(Wo . attn). Each step's result is handed on
    in the I/O dtype. Returns (y [B, 1, d], k_cache', v_cache', new_step).
    """
    B = x.shape[0]
    n = rmsnorm(x, None, eps, out=io)
    q = linear_int8(n, wq, sq, out=io).reshape(B, 1, Hq, D)
    k = linear_int8(n, wk, sk, out=io).reshape(B, 1, Hkv, D)
    v = linear_int8(n, wv, sv, out=io).reshape(B, 1, Hkv, D)
    a, kc, vc, new_step = decode_step(k_cache, v_cache, q, k, v, step, mult, cap, base, io)
    o = linear_int8(a, wo, so, out=io)
    return rmsnorm(o, None, eps, residual=x, out=io), kc, vc, new_step


def chunk_prefill(k_cache, v_cache, q, k_new, v_new, step, mult, cap=30.0, base=10000.0,
                  io="bf16"):
    """A chunk of T new tokens per sequence into a non-empty memory ([ch4] §4.4
    RoPE before the cache write; [ch6] §6.6.1 per-sequence step).

    The pages' mask shapes do not cover T > 1 after a non-empty memory; the
    causal rule is taken on absolute positions: token t of sequence b sits at
    position p = step[b] + t, is rotated there, written to slot p, and attends
    slots [0, p]. Inputs are float64 values already in the I/O dtype. Returns
    (out [B, T, Hq*D], k_cache', v_cache', new_step = step + T).
    """
    B, T = q.shape[:2]
    pos = np.asarray(step, dtype=np.int64).reshape(B, 1) + np.arange(T)
    qr = rope(q, pos, base, out=io)
    kr = rope(k_new, pos, base, out=io)
    kc, vc, new_step = kv_append(k_cache, v_cache, kr, np.asarray(v_new, np.float64), step)
    Tmax = kc.shape[1]
    mask = attention_mask(pos, Tmax, kv_len=new_step)
    o = attention(qr, kc, vc, mask, mult, cap, out=io)
    return o, kc, vc, new_step


def gelu(x):
    """GELU in the tanh form ([ch6] §6.2 calls jax.nn.gelu, whose default is this
    approximation): 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def moe_route(n, w_router, k=2):
    """Router ([ch3] §3.5; [ch2] §2.2): logits n @ W_r with a float32 weight
    matrix [d, E], softmax over the E experts, the k most probable experts.

    Returns (probs [..., E], idx [..., k] int64, gates [..., k]): gates are the
    selected softmax probabilities themselves, not renormalised ([ch2] §2.5.1).
    Ties keep the lower expert index first.
    """
    logits = np.asarray(n, np.float64) @ np.asarray(w_router, np.float64)
    probs = softmax(logits, axis=-1)
    idx = np.argsort(-probs, axis=-1, kind="stable")[..., :k]
    gates = np.take_along_axis(probs, idx, axis=-1)
    return probs, idx, gates


def expert_ffn(n, wg, sg, wv, sv, w1, s1, io="bf16"):
    """One expert, the gated FFN of [ch6] §6.2: (gelu(n Wg) * (n Wv)) W1 with
    int8 Linears (Wg, Wv [d, F]; W1 [F, d]). The two up projections are handed
    on in the I/O dtype, gelu(g) * v is rounded once, the down projection too."""
    g = linear_int8(n, wg, sg, out=io)
    v = linear_int8(n, wv, sv, out=io)
    h = round_to(gelu(g) * v, io)
    return linear_int8(h, w1, s1, out=io)


def moe_sublayer(x, w_router, experts, eps=1e-5, k=2, io="bf16", idx=None):
    """The FFN half of a decoder layer ([ch6] §6.3.1 sandwich norm; [ch2] §2.2):
    n = norm(x); the k routed experts' outputs weighted by their gates and
    summed (rounded once); y = x + norm(sum). No token is dropped (every token
    goes to k experts). `experts` is a list of (wg, sg, wv, sv, w1, s1).
    `idx` ([..., k]) may force the expert choice (for comparisons where the
    router's top-k is tied within rounding). Returns (y, idx, gates)."""
    n = rmsnorm(x, None, eps, out=io)
    probs, idx0, gates = moe_route(n, w_router, k)
    if idx is None:
        idx = idx0
    else:
        idx = np.asarray(idx)
        gates = np.take_along_axis(probs, idx, axis=-1)
    lead = x.shape[:-1]
    nf = n.reshape(-1, n.shape[-1])
    idf = idx.reshape(-1, k)
    gf = gates.reshape(-1, k)
    acc = np.zeros_like(nf)
    for e, ex in enumerate(experts):
        rows, slots = np.nonzero(idf == e)
        if rows.size:
            acc[rows] += gf[rows, slots][:, None] * expert_ffn(nf[rows], *ex, io=io)
    mix = round_to(acc.reshape(*lead, -1), io)
    return rmsnorm(mix, None, eps, residual=x, out=io), idx, gates


def kv_cache_bytes(num_layers, batch, seq_len, num_kv_heads, head_size, elem_bytes=2):
    """[ch6] §6.6.3: K and V, per layer, [B, T, Hkv, D] elements of elem_bytes."""
    return 2 * num_layers * batch * seq_len * num_kv_heads * head_size * elem_bytes
