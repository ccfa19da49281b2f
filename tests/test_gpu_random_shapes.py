"""GPU parity against the fp64 oracle on seeded random shapes: prefill (bf16
MFMA path, optional key padding; fp32 generic path), decode (plain and with the
append fused), chunked prefill after cached prefixes, RMSNorm and the int8
Linears (tiled and few-row), with a few longer cases (prompts up to 1200 rows,
decode batches of 6-20 sequences, prefixes of 1000-4000 slots). The shapes are
drawn once from fixed seeds, so every run checks the same cases; each case
prints its shape in the test id."""
import math

import numpy as np
import pytest

import gqa_inputs as gi
import oracle as orc

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261202)


def _heads():
    hkv = int(_rng.choice([1, 2, 4, 8]))
    return hkv * int(_rng.choice([1, 2, 3, 6])), hkv


def _prefill_cases(n):
    out = []
    for _ in range(n):
        hq, hkv = _heads()
        out.append((int(_rng.integers(1, 4)), int(_rng.integers(1, 201)), hq, hkv,
                    float(_rng.choice([1.0, 4.0])), bool(_rng.integers(0, 2)), int(_rng.integers(0, 1 << 30))))
    return out


def _decode_cases(n):
    out = []
    for _ in range(n):
        hq, hkv = _heads()
        B, Tmax = int(_rng.integers(1, 6)), int(_rng.integers(64, 701))
        lens = [int(x) for x in _rng.integers(1, Tmax + 1, size=B)]
        out.append((hq, hkv, Tmax, lens, int(_rng.integers(0, 1 << 30))))
    return out


def _chunk_cases(n):
    out = []
    for _ in range(n):
        hq, hkv = _heads()
        B, T = int(_rng.integers(1, 5)), int(_rng.integers(1, 101))
        Tmax = T + int(_rng.integers(0, 501))
        offsets = [int(x) for x in _rng.integers(0, Tmax - T + 1, size=B)]
        out.append((hq, hkv, T, Tmax, offsets, int(_rng.integers(0, 1 << 30))))
    return out


PREFILL = _prefill_cases(8)
DECODE = _decode_cases(6)
CHUNK = _chunk_cases(6)

# Longer cases from a stream of their own (the cases above keep their draws):
# prompts up to 1200 rows, batches of decode that cross from grids resident
# at once to larger ones, chunks after prefixes of 1000-4000 slots.
_rng3 = np.random.default_rng(20261204)
for _ in range(3):
    hq, hkv = (lambda h: (h * int(_rng3.choice([1, 2, 3, 6])), h))(int(_rng3.choice([1, 2, 4, 8])))
    PREFILL.append((int(_rng3.integers(1, 3)), int(_rng3.integers(300, 1201)), hq, hkv,
                    float(_rng3.choice([1.0, 4.0])), bool(_rng3.integers(0, 2)), int(_rng3.integers(0, 1 << 30))))
for _ in range(3):
    hq, hkv = (lambda h: (h * int(_rng3.choice([1, 2, 3, 6])), h))(int(_rng3.choice([1, 2, 4, 8])))
    B, Tmax = int(_rng3.integers(6, 21)), int(_rng3.integers(500, 3001))
    DECODE.append((hq, hkv, Tmax, [int(x) for x in _rng3.integers(1, Tmax + 1, size=B)],
                   int(_rng3.integers(0, 1 << 30))))
for _ in range(3):
    hq, hkv = (lambda h: (h * int(_rng3.choice([1, 2, 3, 6])), h))(int(_rng3.choice([1, 2, 4, 8])))
    B, T = int(_rng3.integers(1, 4)), int(_rng3.integers(1, 301))
    Tmax = T + int(_rng3.integers(1000, 4001))
    CHUNK.append((hq, hkv, T, Tmax, [int(x) for x in _rng3.integers(0, Tmax - T + 1, size=B)],
                  int(_rng3.integers(0, 1 << 30))))


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gqa_attention_grok_amd as grok
    import gpu_util
    return grok, gpu_util, torch


@pytest.mark.parametrize("B,T,Hq,Hkv,scale,padded,seed", PREFILL,
                         ids=[f"B{c[0]}-T{c[1]}-Hq{c[2]}-Hkv{c[3]}-x{c[4]:g}-pad{int(c[5])}" for c in PREFILL])
def test_random_prefill_bf16(G, B, T, Hq, Hkv, scale, padded, seed):
    grok, U, torch = G
    D = 128
    mult = scale / math.sqrt(D)
    p = gi.make_prefill_inputs(B, T, Hq, Hkv, D, seed=seed, dtype="bf16", key_pad_frac=0.1 if padded else 0.0)
    pad = p.get("key_valid") if padded else None
    out = torch.empty((B, T, Hq * D), dtype=torch.bfloat16, device="cuda")
    grok.grok_attn_prefill(U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"]), out, mult, 30.0,
                           key_valid=None if pad is None else U.dev(pad))
    to64 = orc.bf16_bits_to_f64
    mask = orc.attention_mask(np.broadcast_to(np.arange(T), (B, T)), T, key_valid=pad)
    ref = orc.attention(to64(p["q"]), to64(p["k"]), to64(p["v"]), mask, mult, 30.0)
    U.assert_bf16_close(U.host(out), ref, f"random prefill B={B} T={T} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("case", range(3))
def test_random_prefill_f32_generic(G, case):
    grok, U, torch = G
    rng = np.random.default_rng(4000 + case)
    D = int(rng.choice([8, 32, 64]))
    hkv = int(rng.choice([1, 2]))
    Hq, B, T = hkv * int(rng.choice([1, 3])), int(rng.integers(1, 3)), int(rng.integers(1, 40))
    p = gi.make_prefill_inputs(B, T, Hq, hkv, D, seed=5000 + case, dtype="f32")
    out = torch.empty((B, T, Hq * D), dtype=torch.float32, device="cuda")
    mult = 1 / math.sqrt(D)
    grok.grok_attn_prefill(U.dev(p["q"]), U.dev(p["k"]), U.dev(p["v"]), out, mult, 30.0)
    mask = orc.attention_mask(np.broadcast_to(np.arange(T), (B, T)), T)
    ref = orc.attention(p["q"].astype(np.float64), p["k"].astype(np.float64), p["v"].astype(np.float64), mask,
                        mult, 30.0)
    U.assert_f32_close(U.host(out), ref, f"random f32 prefill B={B} T={T} Hq={Hq} Hkv={hkv} D={D}")


@pytest.mark.parametrize("Hq,Hkv,Tmax,lens,seed", DECODE,
                         ids=[f"Hq{c[0]}-Hkv{c[1]}-Tmax{c[2]}-B{len(c[3])}" for c in DECODE])
def test_random_decode(G, Hq, Hkv, Tmax, lens, seed):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    B, D = len(lens), 128
    mult = 1 / math.sqrt(D)
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=seed, lengths=lens)
    kv_len = np.asarray(lens, np.int32)
    to64 = orc.bf16_bits_to_f64
    # plain decode over caches that already hold every attended slot
    out = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8, device="cuda")
    grok.grok_attn_decode(U.dev_bf16(p["q"]), U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"]), U.dev(kv_len),
                          out, ws, mult)
    mask = orc.attention_mask((kv_len - 1)[:, None], Tmax, kv_len=kv_len)
    ref = orc.attention(to64(p["q"]), to64(p["k_cache"]), to64(p["v_cache"]), mask, mult, 30.0)
    U.assert_bf16_close(U.host(out), ref, f"random decode lens={lens}")
    # the fused step (RoPE + append of the new token, then attention) is a
    # one-token chunk at offset step[b] for the oracle
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    st = pipe.DecodeStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                         U.dev(p["step"]), mult)
    got = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    ref2, _, _, _ = orc.chunk_prefill(to64(p["k_cache"]), to64(p["v_cache"]), to64(p["q"]), to64(p["k_new"]),
                                      to64(p["v_new"]), p["step"], mult)
    U.assert_bf16_close(got, ref2, f"random fused decode lens={lens}")


@pytest.mark.parametrize("Hq,Hkv,T,Tmax,offsets,seed", CHUNK,
                         ids=[f"Hq{c[0]}-Hkv{c[1]}-T{c[2]}-Tmax{c[3]}-B{len(c[4])}" for c in CHUNK])
def test_random_prefill_chunk(G, Hq, Hkv, T, Tmax, offsets, seed):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    B, D = len(offsets), 128
    mult = 1 / math.sqrt(D)
    p = gi.make_chunk_inputs(B, T, Hq, Hkv, D, Tmax, seed=seed, offsets=offsets)
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    st = pipe.ChunkStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                        U.dev(p["step"]), mult)
    out = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    to64 = orc.bf16_bits_to_f64
    ref, _, _, _ = orc.chunk_prefill(to64(p["k_cache"]), to64(p["v_cache"]), to64(p["q"]), to64(p["k_new"]),
                                     to64(p["v_new"]), p["step"], mult)
    U.assert_bf16_close(out, ref, f"random chunk T={T} offsets={offsets}")


_rng2 = np.random.default_rng(20261203)
NORM = [(int(_rng2.integers(1, 51)), int(_rng2.integers(1, 9001)), bool(_rng2.integers(0, 2)),
         bool(_rng2.integers(0, 2)), str(_rng2.choice(["bf16", "f32"]))) for _ in range(5)]
LINEAR = [(int(_rng2.integers(1, 601)), 8 * int(_rng2.integers(1, 401)), 8 * int(_rng2.integers(1, 301)))
          for _ in range(4)]
GEMV = [(int(_rng2.integers(1, 81)), 8 * int(_rng2.integers(1, 801)),
         tuple(8 * int(n) for n in _rng2.integers(1, 201, size=int(_rng2.integers(1, 4))))) for _ in range(4)]


@pytest.mark.parametrize("rows,d,use_gamma,use_res,dtype", NORM,
                         ids=[f"r{c[0]}-d{c[1]}-g{int(c[2])}-res{int(c[3])}-{c[4]}" for c in NORM])
def test_random_rmsnorm(G, rows, d, use_gamma, use_res, dtype):
    grok, U, torch = G
    g = gi.rng(rows * 7 + d)
    if dtype == "bf16":
        xb, rb = gi.normal_bf16(g, (rows, d)), gi.normal_bf16(g, (rows, d))
        x, r = U.dev_bf16(xb), U.dev_bf16(rb)
        x64, r64 = orc.bf16_bits_to_f64(xb), orc.bf16_bits_to_f64(rb)
    else:
        xf, rf = gi.normal_f32(g, (rows, d)) * 3, gi.normal_f32(g, (rows, d))
        x, r = U.dev(xf), U.dev(rf)
        x64, r64 = xf.astype(np.float64), rf.astype(np.float64)
    gam = g.uniform(0.5, 1.5, d).astype(np.float32) if use_gamma else None
    y = torch.empty_like(x)
    grok.grok_rmsnorm(x, y, gamma=U.dev(gam) if use_gamma else None, residual=r if use_res else None)
    ref = r64 + orc.rmsnorm(x64, gam, 1e-5, out=dtype) if use_res else orc.rmsnorm(x64, gam, 1e-5)
    if dtype == "bf16":
        U.assert_bf16_close(U.host(y), ref, f"random rmsnorm rows={rows} d={d}")
    else:
        U.assert_f32_close(U.host(y), ref, f"random rmsnorm rows={rows} d={d}")


@pytest.mark.parametrize("M,K,N", LINEAR, ids=[f"M{c[0]}-K{c[1]}-N{c[2]}" for c in LINEAR])
def test_random_linear_int8(G, M, K, N):
    grok, U, torch = G
    g = gi.rng(M * 3 + K + N)
    xb, w = gi.normal_bf16(g, (M, K)), gi.int8_uniform(g, (K, N))
    s = (0.02 / 127 * g.uniform(0.5, 1.5, N)).astype(np.float32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    grok.grok_linear_int8(U.dev_bf16(xb), U.dev(w), U.dev(s), y)
    U.assert_bf16_close(U.host(y), orc.linear_int8(orc.bf16_bits_to_f64(xb), w, s), f"random linear M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,Ns", GEMV, ids=[f"M{c[0]}-K{c[1]}-N{'_'.join(map(str, c[2]))}" for c in GEMV])
def test_random_gemv(G, M, K, Ns):
    grok, U, torch = G
    g = gi.rng(M * 5 + K + sum(Ns))
    xb = gi.normal_bf16(g, (M, K))
    ws = [gi.int8_uniform(g, (K, n)) for n in Ns]
    ss = [(0.02 / 127 * g.uniform(0.5, 1.5, n)).astype(np.float32) for n in Ns]
    wp = [grok.grok_linear_int8_pack(U.dev(w)) for w in ws]
    ys = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in Ns]
    grok.grok_linear_int8_gemv(U.dev_bf16(xb), wp, [U.dev(s) for s in ss], ys)
    x64 = orc.bf16_bits_to_f64(xb)
    for p in range(len(Ns)):
        U.assert_bf16_close(U.host(ys[p]), orc.linear_int8(x64, ws[p], ss[p]), f"random gemv M={M} K={K} matrix {p}")
