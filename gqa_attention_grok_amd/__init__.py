"""Python binding of ``libgrokattn.so`` (the gfx950 Grok-1 attention core).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream of torch to the C ABI declared in
``include/grok_attn.h`` and raises ``GrokError`` on a non-zero status. All
computation happens in the library's HIP kernels; there is no fallback. If
the shared library has not been built, importing this package raises.

Tensors are torch tensors on the GPU: bf16 data as ``torch.bfloat16``, fp32
as ``torch.float32``, int8 weights as ``torch.int8``, positions/lengths as
``torch.int32``, key masks as ``torch.uint8``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GrokError", "LIB_PATH", "lib", "GROK_BF16", "GROK_F32",
    "grok_abi_version", "grok_status_string", "grok_last_error",
    "grok_rmsnorm", "grok_linear_int8", "grok_linear_int8_packed_bytes",
    "grok_linear_int8_pack", "grok_linear_int8_gemv", "grok_decode_qkv", "grok_decode_out",
    "grok_decode_out_workspace_bytes", "grok_rope", "grok_kv_append",
    "grok_attn_prefill", "grok_attn_prefill_rope", "grok_attn_prefill_rope_workspace_bytes",
    "grok_attn_prefill_chunk", "grok_attn_decode", "grok_attn_decode_append",
    "grok_attn_decode_append_noalloc", "grok_attn_decode_append_noalloc_max_bytes",
    "grok_attn_decode_workspace_bytes", "grok_moe_workspace_bytes", "grok_moe_interleave",
    "grok_moe_route", "grok_moe_ffn", "grok_prefill_qkv_workspace_bytes", "grok_prefill_qkv",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgrokattn.so")
GROK_BF16, GROK_F32 = 0, 1
GROK_OK, GROK_EHIP, GROK_ENOMEM, GROK_EINVAL, GROK_ERANGE = 0, -5, -12, -22, -34

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python gqa_attention_grok_amd/build.py` "
        "(there is no non-HIP fallback)")

lib = ctypes.CDLL(LIB_PATH)

_p, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_PROTOS = {
    "grok_abi_version": (_i, []),
    "grok_status_string": (ctypes.c_char_p, [_i]),
    "grok_last_error": (ctypes.c_char_p, []),
    "grok_rmsnorm": (_i, [_p, _p, _p, _p, _i64, _i, _f, _i, _p]),
    "grok_linear_int8": (_i, [_p, _p, _p, _p, _i64, _i, _i, _p]),
    "grok_linear_int8_packed_bytes": (_sz, [_i, _i]),
    "grok_linear_int8_pack": (_i, [_p, _p, _i, _i, _p]),
    "grok_linear_int8_gemv": (_i, [_p, _i, _p, _p, _p, _p, _i64, _i, _p]),
    "grok_decode_qkv": (_i, [_p, _p, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                             _i, _i, _i, _i, _i, _i, _f, _p]),
    "grok_decode_out_workspace_bytes": (_sz, [_i, _i, _i]),
    "grok_decode_out": (_i, [_p, _p, _p, _p, _f, _p, _p, _p, _sz, _i, _i, _i, _p]),
    "grok_rope": (_i, [_p, _i, _i, _i, _i, _p, _f, _i, _p]),
    "grok_kv_append": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _p]),
    "grok_attn_prefill": (_i, [_p, _p, _p, _i64, _p, _p, _i, _i, _i, _i, _i, _f, _f, _i, _p]),
    "grok_attn_prefill_rope_workspace_bytes": (_sz, [_i, _i]),
    "grok_attn_prefill_rope": (_i, [_p, _p, _p, _i64, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _f, _f, _f, _p]),
    "grok_attn_decode": (_i, [_p, _p, _p, _p, _p, _p, _sz, _p, _i, _i, _i, _i, _i, _f, _f, _p]),
    "grok_attn_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "grok_attn_prefill_chunk": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _f, _p]),
    "grok_attn_decode_append": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _i, _i, _i, _i, _i,
                                     _f, _f, _f, _p]),
    "grok_attn_decode_append_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i,
                                             _f, _f, _f, _p]),
    "grok_attn_decode_append_noalloc_max_bytes": (_sz, []),
    "grok_moe_workspace_bytes": (_sz, [_i64, _i, _i, _i, _i]),
    "grok_prefill_qkv_workspace_bytes": (_sz, [_i, _i]),
    "grok_prefill_qkv": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _i,
                              _i, _f, _p]),
    "grok_moe_interleave": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _p]),
    "grok_moe_route": (_i, [_p, _p, _p, _p, _i64, _i, _i, _i, _p]),
    "grok_moe_ffn": (_i, [_p, _p, _i, _i, _p, _p, _p, _p, _i64, _i, _i, _f, _p, _p, _p, _sz, _p, _p]),
}
for _name, (_res, _args) in _PROTOS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class GrokError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.grok_last_error().decode() or lib.grok_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def _check(status: int, where: str):
    if status != GROK_OK:
        raise GrokError(status, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return GROK_BF16
    if t.dtype == torch.float32:
        return GROK_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def grok_abi_version() -> int:
    return lib.grok_abi_version()


def grok_status_string(status: int) -> str:
    return lib.grok_status_string(status).decode()


def grok_last_error() -> str:
    return lib.grok_last_error().decode()


def grok_rmsnorm(x, y, gamma=None, residual=None, eps=1e-5):
    """y[..., d] = [residual +] gamma * x / sqrt(mean(x^2) + eps) over the last axis."""
    _need(x, "x")
    _need(y, "y", x.dtype)
    _need(gamma, "gamma", torch.float32)
    _need(residual, "residual", x.dtype)
    d = x.shape[-1]
    _check(lib.grok_rmsnorm(_ptr(x), _ptr(gamma), _ptr(residual), _ptr(y), x.numel() // d, d,
                            eps, _dtype_code(x), _stream(x)), "grok_rmsnorm")
    return y


def grok_linear_int8(x, w, scales, y):
    """y [M, N] = x [M, K] @ (w [K, N] int8 * scales [N])."""
    _need(x, "x", torch.bfloat16)
    _need(w, "w", torch.int8, 2)
    _need(scales, "scales", torch.float32, 1)
    _need(y, "y", torch.bfloat16)
    K, N = w.shape
    _check(lib.grok_linear_int8(_ptr(x), _ptr(w), _ptr(scales), _ptr(y), x.numel() // K, K, N,
                                _stream(x)), "grok_linear_int8")
    return y


def grok_linear_int8_packed_bytes(K, N) -> int:
    return lib.grok_linear_int8_packed_bytes(K, N)


def grok_linear_int8_pack(w, w_packed=None):
    """Packed form of the int8 weights w [K, N] for grok_linear_int8_gemv (a new
    int8 tensor of grok_linear_int8_packed_bytes(K, N) bytes unless one is given)."""
    _need(w, "w", torch.int8, 2)
    K, N = w.shape
    nbytes = grok_linear_int8_packed_bytes(K, N)
    if w_packed is None:
        w_packed = torch.empty(nbytes, dtype=torch.int8, device=w.device)
    _need(w_packed, "w_packed", torch.int8)
    if w_packed.numel() != nbytes:
        raise ValueError(f"w_packed must hold {nbytes} bytes")
    _check(lib.grok_linear_int8_pack(_ptr(w), _ptr(w_packed), K, N, _stream(w)), "grok_linear_int8_pack")
    return w_packed


def grok_linear_int8_gemv(x, w_packed, scales, ys):
    """ys[p] [M, N_p] = x [M, K] @ (W_p * scales[p]) for up to three matrices that
    share x, in one launch; w_packed[p] is grok_linear_int8_pack(W_p)."""
    _need(x, "x", torch.bfloat16)
    if not (len(w_packed) == len(scales) == len(ys)):
        raise ValueError("w_packed, scales and ys must have the same length")
    K = x.shape[-1]
    M = x.numel() // K
    Ns = []
    for p, (w, s, y) in enumerate(zip(w_packed, scales, ys)):
        _need(w, f"w_packed[{p}]", torch.int8)
        _need(s, f"scales[{p}]", torch.float32, 1)
        _need(y, f"ys[{p}]", torch.bfloat16)
        N = s.shape[0]
        if y.numel() != M * N or w.numel() != grok_linear_int8_packed_bytes(K, N):
            raise ValueError(f"matrix {p}: sizes do not match x [{M}, {K}] and {N} channels")
        Ns.append(N)
    n = len(Ns)
    wa = (_p * n)(*[_ptr(w) for w in w_packed])
    sa = (_p * n)(*[_ptr(s) for s in scales])
    ya = (_p * n)(*[_ptr(y) for y in ys])
    na = (_i * n)(*Ns)
    _check(lib.grok_linear_int8_gemv(_ptr(x), n, ctypes.cast(wa, _p), ctypes.cast(sa, _p),
                                     ctypes.cast(ya, _p), ctypes.cast(na, _p), M, K, _stream(x)),
           "grok_linear_int8_gemv")
    return ys


def grok_decode_qkv(x, wq_packed, sq, wk_packed, sk, wv_packed, sv, q_out, k_cache, v_cache,
                    step, new_step=None, status=None, prenorm=False, gamma=None, eps=1e-5,
                    rope_base=10000.0):
    """One new token per sequence: [n = rmsnorm(x)]; q_out = rope(n Wq) at step[b];
    k_cache/v_cache slot step[b] = rope(n Wk), n Wv; new_step = step + 1."""
    _need(x, "x", torch.bfloat16)
    _need(q_out, "q_out", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    for t, n in ((wq_packed, "wq_packed"), (wk_packed, "wk_packed"), (wv_packed, "wv_packed")):
        _need(t, n, torch.int8)
    for t, n in ((sq, "sq"), (sk, "sk"), (sv, "sv")):
        _need(t, n, torch.float32, 1)
    _need(step, "step", torch.int32, 1)
    _need(new_step, "new_step", torch.int32, 1)
    _need(status, "status", torch.int32)
    _need(gamma, "gamma", torch.float32, 1)
    B, Tmax, Hkv, D = k_cache.shape
    d = x.shape[-1]
    Hq = sq.shape[0] // D
    if x.numel() != B * d or q_out.numel() != B * Hq * D or step.numel() != B:
        raise ValueError("decode_qkv: x, q_out and step must hold B rows")
    for w_, N in ((wq_packed, Hq * D), (wk_packed, Hkv * D), (wv_packed, Hkv * D)):
        if w_.numel() != grok_linear_int8_packed_bytes(d, N):
            raise ValueError("decode_qkv: packed weights do not match the sizes")
    _check(lib.grok_decode_qkv(_ptr(x), _ptr(gamma), eps, 1 if prenorm else 0, _ptr(wq_packed), _ptr(sq),
                               _ptr(wk_packed), _ptr(sk), _ptr(wv_packed), _ptr(sv), _ptr(q_out),
                               _ptr(k_cache), _ptr(v_cache), _ptr(step), _ptr(new_step), _ptr(status),
                               B, d, Tmax, Hq, Hkv, D, rope_base, _stream(x)), "grok_decode_qkv")
    return q_out


def grok_rope(x, offset=None, base=10000.0):
    """In-place RoPE of x [B, T, H, D] at positions offset[b] + t."""
    _need(x, "x", ndim=4)
    _need(offset, "offset", torch.int32, 1)
    B, T, H, D = x.shape
    _check(lib.grok_rope(_ptr(x), B, T, H, D, _ptr(offset), base, _dtype_code(x), _stream(x)),
           "grok_rope")
    return x


def grok_decode_out_workspace_bytes(B, d_in, d_out):
    return int(lib.grok_decode_out_workspace_bytes(B, d_in, d_out))


def grok_decode_out(attn, wo_packed, so, residual, y, workspace, gamma=None, eps=1e-5):
    """y = residual + norm(attn @ (Wo * so)) for one token per sequence (the
    attention sub-layer's back half); one launch for up to 4 rows. The
    workspace (uint8, grok_decode_out_workspace_bytes) must be zeroed once
    before its first use; each call leaves it ready for the next."""
    _need(attn, "attn", torch.bfloat16)
    _need(wo_packed, "wo_packed", torch.int8)
    _need(so, "so", torch.float32, 1)
    _need(gamma, "gamma", torch.float32, 1)
    _need(residual, "residual", torch.bfloat16)
    _need(y, "y", torch.bfloat16)
    _need(workspace, "workspace")
    d_out = so.shape[0]
    B = residual.numel() // d_out
    d_in = attn.numel() // B
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.grok_decode_out(_ptr(attn), _ptr(wo_packed), _ptr(so), _ptr(gamma), eps, _ptr(residual), _ptr(y),
                               _ptr(workspace), ws_bytes, B, d_in, d_out, _stream(attn)), "grok_decode_out")
    return y


def grok_kv_append(k_cache, v_cache, k_new, v_new, step, q_inout=None, new_step=None,
                   status=None, rope_base=10000.0):
    """RoPE q/k at step[b] + t, write k/v into the caches at that slot."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, torch.bfloat16, 4)
    _need(q_inout, "q_inout", torch.bfloat16, 4)
    _need(step, "step", torch.int32, 1)
    _need(new_step, "new_step", torch.int32, 1)
    _need(status, "status", torch.int32)
    B, Tmax, Hkv, D = k_cache.shape
    T = k_new.shape[1]
    Hq = q_inout.shape[2] if q_inout is not None else 0
    _check(lib.grok_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(q_inout),
                              _ptr(step), _ptr(new_step), _ptr(status), B, T, Tmax, Hq, Hkv, D,
                              rope_base, _stream(k_cache)), "grok_kv_append")


def grok_attn_prefill(q, k, v, out, attn_mult, softcap=30.0, key_valid=None):
    """Causal GQA: q [B,T,Hq,D], k/v [B,kv_rows,Hkv,D] (kv_rows >= T), out [B,T,Hq*D]."""
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    _need(out, "out", q.dtype)
    _need(key_valid, "key_valid", torch.uint8, 2)
    B, T, Hq, D = q.shape
    kv_rows, Hkv = k.shape[1], k.shape[2]
    _check(lib.grok_attn_prefill(_ptr(q), _ptr(k), _ptr(v), kv_rows, _ptr(key_valid), _ptr(out),
                                 B, T, Hq, Hkv, D, attn_mult, softcap, _dtype_code(q), _stream(q)),
           "grok_attn_prefill")
    return out


def grok_attn_prefill_rope_workspace_bytes(T, D=128) -> int:
    return int(lib.grok_attn_prefill_rope_workspace_bytes(T, D))


def grok_attn_prefill_rope(q, k, v, out, workspace, attn_mult, softcap=30.0, key_valid=None, rope_base=10000.0):
    """Causal GQA with q rotated at positions 0..T-1 inside the kernel (q is not
    modified; k must be rotated already); bf16, D = 128."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(out, "out", torch.bfloat16)
    _need(workspace, "workspace")
    _need(key_valid, "key_valid", torch.uint8, 2)
    B, T, Hq, D = q.shape
    kv_rows, Hkv = k.shape[1], k.shape[2]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.grok_attn_prefill_rope(_ptr(q), _ptr(k), _ptr(v), kv_rows, _ptr(key_valid), _ptr(out),
                                      _ptr(workspace), ws_bytes, B, T, Hq, Hkv, D, attn_mult, softcap, rope_base,
                                      _stream(q)), "grok_attn_prefill_rope")
    return out


def grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D) -> int:
    return lib.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D)


def grok_attn_decode(q, k_cache, v_cache, kv_len, out, workspace, attn_mult, softcap=30.0,
                     status=None):
    """One-token GQA against the cache slots [0, kv_len[b]); q [B,1,Hq,D], out [B,1,Hq*D]."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(kv_len, "kv_len", torch.int32, 1)
    _need(out, "out", torch.bfloat16)
    _need(workspace, "workspace")
    _need(status, "status", torch.int32)
    B, _, Hq, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.grok_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(out),
                                _ptr(workspace), ws_bytes, _ptr(status), B, Tmax, Hq, Hkv, D,
                                attn_mult, softcap, _stream(q)), "grok_attn_decode")
    return out


def grok_attn_decode_append(q, k_new, v_new, k_cache, v_cache, step, out, workspace, attn_mult,
                            softcap=30.0, new_step=None, q_out=None, status=None, rope_base=10000.0):
    """RoPE q and the new k at step[b], write k/v to slot step[b], attend slots
    [0, step[b]]: one decode step in one call (q itself is not modified)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_new, "k_new", torch.bfloat16, 4)
    _need(v_new, "v_new", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(step, "step", torch.int32, 1)
    _need(out, "out", torch.bfloat16)
    _need(workspace, "workspace")
    _need(new_step, "new_step", torch.int32, 1)
    _need(q_out, "q_out", torch.bfloat16)
    _need(status, "status", torch.int32)
    B, _, Hq, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.grok_attn_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(step), _ptr(new_step), _ptr(q_out), _ptr(out), _ptr(workspace),
                                       ws_bytes, _ptr(status), B, Tmax, Hq, Hkv, D, attn_mult, softcap,
                                       rope_base, _stream(q)), "grok_attn_decode_append")
    return out


def grok_attn_decode_append_noalloc_max_bytes():
    return int(lib.grok_attn_decode_append_noalloc_max_bytes())


def grok_attn_decode_append_noalloc(q, k_new, v_new, k_cache, v_cache, step, out, attn_mult, softcap=30.0,
                                    new_step=None, q_out=None, status=None, rope_base=10000.0):
    """grok_attn_decode_append without a workspace: the library's per-GPU
    scratch array holds the split partials (no device allocation per call;
    calls that overlap on one GPU race)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_new, "k_new", torch.bfloat16, 4)
    _need(v_new, "v_new", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(step, "step", torch.int32, 1)
    _need(out, "out", torch.bfloat16)
    _need(new_step, "new_step", torch.int32, 1)
    _need(q_out, "q_out", torch.bfloat16)
    _need(status, "status", torch.int32)
    B, _, Hq, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(lib.grok_attn_decode_append_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(step), _ptr(new_step), _ptr(q_out), _ptr(out), _ptr(status),
                                               B, Tmax, Hq, Hkv, D, attn_mult, softcap, rope_base, _stream(q)),
           "grok_attn_decode_append_noalloc")
    return out


def grok_attn_prefill_chunk(q, k_cache, v_cache, offset, out, attn_mult, softcap=30.0, status=None):
    """Chunk of T tokens per sequence at positions offset[b] + t, attending cache
    slots [0, offset[b] + t]; q [B,T,Hq,D] rotated, out [B,T,Hq*D]."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(offset, "offset", torch.int32, 1)
    _need(out, "out", torch.bfloat16)
    _need(status, "status", torch.int32)
    B, T, Hq, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(lib.grok_attn_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(offset), _ptr(out),
                                       _ptr(status), B, T, Tmax, Hq, Hkv, D, attn_mult, softcap, _stream(q)),
           "grok_attn_prefill_chunk")
    return out


def grok_moe_workspace_bytes(T, d, F, E, k) -> int:
    return lib.grok_moe_workspace_bytes(T, d, F, E, k)


def grok_moe_interleave(wg, sg, wv, sv, wgv=None, sgv=None):
    """Gate and value up-projection weights of one expert side by side in blocks
    of four columns (the form grok_moe_ffn reads): wgv [d, 2F], sgv [2F]."""
    _need(wg, "wg", torch.int8, 2)
    _need(wv, "wv", torch.int8, 2)
    _need(sg, "sg", torch.float32, 1)
    _need(sv, "sv", torch.float32, 1)
    d, F = wg.shape
    if wv.shape != (d, F) or sg.shape != (F,) or sv.shape != (F,):
        raise ValueError("wg, wv [d, F] and sg, sv [F] must match")
    if wgv is None:
        wgv = torch.empty(d, 2 * F, dtype=torch.int8, device=wg.device)
    if sgv is None:
        sgv = torch.empty(2 * F, dtype=torch.float32, device=wg.device)
    _need(wgv, "wgv", torch.int8)
    _need(sgv, "sgv", torch.float32)
    if wgv.numel() != 2 * d * F or sgv.numel() != 2 * F:
        raise ValueError("wgv must hold d*2F bytes and sgv 2F floats")
    _check(lib.grok_moe_interleave(_ptr(wg), _ptr(sg), _ptr(wv), _ptr(sv), _ptr(wgv), _ptr(sgv), d, F,
                                   _stream(wg)), "grok_moe_interleave")
    return wgv, sgv


def grok_moe_route(n, w_router, idx, gates):
    """idx, gates [T, k] = the k most probable experts of softmax(n @ w_router)
    (fp32) and their probabilities; n [T, d] bf16 normalised rows."""
    _need(n, "n", torch.bfloat16)
    _need(w_router, "w_router", torch.float32, 2)
    _need(idx, "idx", torch.int32)
    _need(gates, "gates", torch.float32)
    d, E = w_router.shape
    T = n.numel() // d
    k = idx.shape[-1]
    if idx.numel() != T * k or gates.numel() != T * k:
        raise ValueError("idx and gates must be [T, k]")
    _check(lib.grok_moe_route(_ptr(n), _ptr(w_router), _ptr(idx), _ptr(gates), T, d, E, k, _stream(n)),
           "grok_moe_route")
    return idx, gates


def grok_moe_ffn(x, w_router, wgv, sgv, w1, s1, out, workspace, k=2, eps=1e-5, idx=None, gates=None):
    """out [T, d] = x + norm(sum over the k routed experts of gate * expert(norm(x)))
    with GeGLU experts (wgv[e], sgv[e] from grok_moe_interleave; w1[e] [F, d],
    s1[e] [d]); idx, gates [T, k] optional outputs of the routing."""
    _need(x, "x", torch.bfloat16)
    _need(out, "out", torch.bfloat16)
    _need(w_router, "w_router", torch.float32, 2)
    _need(workspace, "workspace")
    _need(idx, "idx", torch.int32)
    _need(gates, "gates", torch.float32)
    d, E = w_router.shape
    T = x.numel() // d
    if out.numel() != T * d:
        raise ValueError("out must match x")
    if not (len(wgv) == len(sgv) == len(w1) == len(s1) == E):
        raise ValueError(f"need {E} experts' weights")
    F = w1[0].shape[0]
    for e in range(E):
        _need(wgv[e], f"wgv[{e}]", torch.int8)
        _need(sgv[e], f"sgv[{e}]", torch.float32, 1)
        _need(w1[e], f"w1[{e}]", torch.int8, 2)
        _need(s1[e], f"s1[{e}]", torch.float32, 1)
        if wgv[e].numel() != 2 * d * F or sgv[e].numel() != 2 * F or tuple(w1[e].shape) != (F, d) \
                or s1[e].numel() != d:
            raise ValueError(f"expert {e}: weight sizes do not match d={d} F={F}")
    for t, name in ((idx, "idx"), (gates, "gates")):
        if t is not None and t.numel() != T * k:
            raise ValueError(f"{name} must be [T, k]")
    arr = lambda ts: ctypes.cast((_p * E)(*[_ptr(t) for t in ts]), _p)
    _check(lib.grok_moe_ffn(_ptr(x), _ptr(w_router), E, k, arr(wgv), arr(sgv), arr(w1), arr(s1), T, d, F,
                            eps, _ptr(idx), _ptr(gates), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _ptr(out), _stream(x)),
           "grok_moe_ffn")
    return out


def grok_prefill_qkv_workspace_bytes(Tmax, D=128) -> int:
    return lib.grok_prefill_qkv_workspace_bytes(Tmax, D)


def grok_prefill_qkv(x, wq, sq, wk, sk, wv, sv, q_out, k_cache, v_cache, workspace, step=None, new_step=None,
                     status=None, rope_base=10000.0):
    """T rows per sequence in one launch: q_out = rope(x Wq) at step[b] + t; the
    cache slots step[b] + t get rope(x Wk) and x Wv (step None: positions t)."""
    _need(x, "x", torch.bfloat16, 3)
    for t, n in ((wq, "wq"), (wk, "wk"), (wv, "wv")):
        _need(t, n, torch.int8, 2)
    for t, n in ((sq, "sq"), (sk, "sk"), (sv, "sv")):
        _need(t, n, torch.float32, 1)
    _need(q_out, "q_out", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(workspace, "workspace")
    _need(step, "step", torch.int32, 1)
    _need(new_step, "new_step", torch.int32, 1)
    _need(status, "status", torch.int32)
    B, T, d = x.shape
    Hq, D = q_out.shape[2], q_out.shape[3]
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(q_out.shape[:2]) != (B, T) or tuple(wq.shape) != (d, Hq * D) or tuple(wk.shape) != (d, Hkv * D) \
            or tuple(wv.shape) != (d, Hkv * D) or k_cache.shape != v_cache.shape or k_cache.shape[0] != B:
        raise ValueError("prefill_qkv: shapes do not match")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.grok_prefill_qkv(_ptr(x), _ptr(wq), _ptr(sq), _ptr(wk), _ptr(sk), _ptr(wv), _ptr(sv), _ptr(q_out),
                                _ptr(k_cache), _ptr(v_cache), _ptr(step), _ptr(new_step), _ptr(status),
                                _ptr(workspace), ws_bytes, B, T, d, Tmax, Hq, Hkv, D, rope_base, _stream(x)),
           "grok_prefill_qkv")
    return q_out
