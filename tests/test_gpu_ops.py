"""GPU parity of every C-ABI entry point against the fp64 oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails,
plus the edge cases (empty, ragged, degenerate masks, out-of-range positions)."""
import math

import numpy as np
import pytest

import gqa_inputs as gi
import oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gqa_attention_grok_amd as grok
    import gpu_util
    return grok, gpu_util, torch


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rows,d,use_gamma,use_res,dtype", [
    (37, 6144, False, False, "bf16"),
    (37, 6144, True, True, "bf16"),
    (5, 100, True, True, "bf16"),      # row not a multiple of the vector width
    (2, 8200, False, True, "bf16"),    # row wider than the register-resident path
    (9, 64, True, False, "f32"),
    (3, 6, False, True, "f32"),
])
def test_rmsnorm(G, rows, d, use_gamma, use_res, dtype):
    grok, U, torch = G
    g = gi.rng(10 + d)
    if dtype == "bf16":
        xb, rb = gi.normal_bf16(g, (rows, d)), gi.normal_bf16(g, (rows, d))
        x, r = U.dev_bf16(xb), U.dev_bf16(rb)
        x64, r64 = orc.bf16_bits_to_f64(xb), orc.bf16_bits_to_f64(rb)
    else:
        x64 = gi.normal_f32(g, (rows, d)) * 3
        r64 = gi.normal_f32(g, (rows, d))
        x, r = U.dev(x64), U.dev(r64)
        x64, r64 = x64.astype(np.float64), r64.astype(np.float64)
    gam = g.uniform(0.5, 1.5, d).astype(np.float32) if use_gamma else None
    y = torch.empty_like(x)
    grok.grok_rmsnorm(x, y, gamma=U.dev(gam) if use_gamma else None, residual=r if use_res else None)
    if use_res:  # the normalised row is handed on rounded, then added exactly
        ref = r64 + orc.rmsnorm(x64, gam, 1e-5, out=dtype)
    else:
        ref = orc.rmsnorm(x64, gam, 1e-5)
    if dtype == "bf16":
        U.assert_bf16_close(U.host(y), ref, "rmsnorm")
    else:
        U.assert_f32_close(U.host(y), ref, "rmsnorm")


def test_rmsnorm_in_place_and_empty(G):
    grok, U, torch = G
    xb = gi.normal_bf16(gi.rng(3), (4, 6144))
    x = U.dev_bf16(xb)
    grok.grok_rmsnorm(x, x)
    U.assert_bf16_close(U.host(x), orc.rmsnorm(orc.bf16_bits_to_f64(xb)), "in place")
    e = torch.empty((0, 6144), dtype=torch.bfloat16, device="cuda")
    grok.grok_rmsnorm(e, e)


# --------------------------------------------------------------------------
# int8 Linear
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,N,distinct", [
    (300, 6144, 1024, True),   # ragged rows, several K steps
    (130, 40, 24, True),       # K tail inside one step, partial channel tile
    (1, 8, 8, False),
    (257, 512, 6144, True),
])
def test_linear_int8(G, M, K, N, distinct):
    grok, U, torch = G
    g = gi.rng(M + K + N)
    xb = gi.normal_bf16(g, (M, K))
    w = gi.int8_uniform(g, (K, N))
    s = (0.02 / 127 * g.uniform(0.5, 1.5, N) if distinct else np.full(N, 0.02 / 127)).astype(np.float32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    grok.grok_linear_int8(U.dev_bf16(xb), U.dev(w), U.dev(s), y)
    ref = orc.linear_int8(orc.bf16_bits_to_f64(xb), w, s)
    U.assert_bf16_close(U.host(y), ref, "linear_int8")


def test_linear_int8_scale_axis_and_empty(G):
    grok, U, torch = G
    K, N = 64, 16
    w = np.zeros((K, N), np.int8)
    w[np.arange(N) * 3, np.arange(N)] = 127  # channel n reads input 3n
    s = (np.arange(1, N + 1) / 127).astype(np.float32)
    xb = gi.normal_bf16(gi.rng(4), (5, K))
    y = torch.empty((5, N), dtype=torch.bfloat16, device="cuda")
    grok.grok_linear_int8(U.dev_bf16(xb), U.dev(w), U.dev(s), y)
    x64 = orc.bf16_bits_to_f64(xb)
    ref = x64[:, np.arange(N) * 3] * 127 * s.astype(np.float64)
    U.assert_bf16_close(U.host(y), ref, "column selection")
    # scales taken along the input axis instead would be off by large factors
    wrong = x64[:, np.arange(N) * 3] * 127 * s[np.arange(N) * 3 % N].astype(np.float64)
    assert np.max(np.abs(U.host(y) - wrong)) > 0.1
    e = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    grok.grok_linear_int8(e, U.dev(w), U.dev(s), torch.empty((0, N), dtype=torch.bfloat16, device="cuda"))


def _packed_reference(w):
    """The packed layout restated with NumPy index arithmetic: tile (j, i) at
    (j * KP + i) * 1024, byte 16*l + 8*h + e = w[64i + 32h + 8(l//16) + e, 16j + l%16]."""
    K, N = w.shape
    KP, NP = -(-K // 64), -(-N // 16)
    wpad = np.zeros((KP * 64, NP * 16), np.int8)
    wpad[:K, :N] = w
    # [j, i, l, h, e] -> w[64i + 32h + 8(l//16) + e, 16j + l%16]
    j, i_, l, h, e = np.meshgrid(np.arange(NP), np.arange(KP), np.arange(64), np.arange(2), np.arange(8),
                                 indexing="ij")
    return wpad[64 * i_ + 32 * h + 8 * (l // 16) + e, 16 * j + l % 16].reshape(-1)


@pytest.mark.parametrize("K,N", [(64, 16), (1000, 136), (8, 8), (6144, 1024)])
def test_linear_int8_pack_layout(G, K, N):
    grok, U, torch = G
    w = gi.int8_uniform(gi.rng(K + N), (K, N))
    wp = grok.grok_linear_int8_pack(U.dev(w))
    np.testing.assert_array_equal(wp.cpu().numpy(), _packed_reference(w))


@pytest.mark.parametrize("M,K,Ns", [
    (1, 6144, (6144, 1024, 1024)),  # one token's Q|K|V: 256 workgroups of 32 channels
    (4, 6144, (6144,)),             # four rows
    (2, 1000, (136, 8, 1024)),      # ragged K and channel blocks
    (3, 8, (8,)),                   # the smallest shape
    (17, 6144, (6144, 1024, 1024)), # two row tiles
    (32, 6144, (6144,)),
    (17, 200, (264,)),
    (70, 512, (128, 256)),          # more than 32 rows: 32 + 32 + 6
    (34, 96, (1024, 24)),           # 32 + 2, a block with half its channels
])
def test_linear_int8_gemv(G, M, K, Ns):
    grok, U, torch = G
    g = gi.rng(7 * M + K + sum(Ns))
    xb = gi.normal_bf16(g, (M, K))
    ws = [gi.int8_uniform(g, (K, n)) for n in Ns]
    ss = [(0.02 / 127 * g.uniform(0.5, 1.5, n)).astype(np.float32) for n in Ns]
    x = U.dev_bf16(xb)
    wp = [grok.grok_linear_int8_pack(U.dev(w)) for w in ws]
    ds = [U.dev(s) for s in ss]
    ys = [torch.empty((M, n), dtype=torch.bfloat16, device="cuda") for n in Ns]
    print(f"gemv M={M} K={K} Ns={Ns}", flush=True)
    grok.grok_linear_int8_gemv(x, wp, ds, ys)
    x64 = orc.bf16_bits_to_f64(xb)
    first = [U.bits(y).copy() for y in ys]
    for p in range(len(Ns)):
        U.assert_bf16_close(U.host(ys[p]), orc.linear_int8(x64, ws[p], ss[p]), f"gemv matrix {p}")
    # a second call gives the same bits (the sums are taken in a fixed order)
    for y in ys:
        y.fill_(0)
    grok.grok_linear_int8_gemv(x, wp, ds, ys)
    for p in range(len(Ns)):
        np.testing.assert_array_equal(U.bits(ys[p]), first[p])


def test_linear_int8_gemv_matches_tiled_kernel_and_empty(G):
    """The few-row product and the tiled product compute the same sums in a
    different order: equal to within an fp32 rounding of the bf16 result."""
    grok, U, torch = G
    M, K, N = 8, 6144, 1024
    g = gi.rng(77)
    xb = gi.normal_bf16(g, (M, K))
    w = U.dev(gi.int8_uniform(g, (K, N)))
    s = U.dev(np.full(N, 0.02 / 127, np.float32))
    x = U.dev_bf16(xb)
    a = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    wp = grok.grok_linear_int8_pack(w)
    grok.grok_linear_int8_gemv(x, [wp], [s], [a])
    grok.grok_linear_int8(x, w, s, b)
    d = np.abs(U.host(a) - U.host(b))
    ulp = np.abs(U.host(b)) * 2.0 ** -7 + 1e-30
    assert np.all(d <= ulp), float((d / ulp).max())
    e = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    grok.grok_linear_int8_gemv(e, [wp], [s], [torch.empty((0, N), dtype=torch.bfloat16, device="cuda")])


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dtype,offsets", [
    ((2, 37, 5, 128), "bf16", [0, 8000]),
    ((1, 16, 6, 32), "f32", None),
    ((3, 4, 2, 6), "f32", [5, 0, 8191]),   # pair count not a multiple of the vector width
    ((1, 3, 48, 128), "bf16", [8189]),
])
def test_rope(G, shape, dtype, offsets):
    grok, U, torch = G
    g = gi.rng(sum(shape))
    B, T = shape[:2]
    if dtype == "bf16":
        xb = gi.normal_bf16(g, shape)
        x, x64 = U.dev_bf16(xb), orc.bf16_bits_to_f64(xb)
    else:
        xf = gi.normal_f32(g, shape)
        x, x64 = U.dev(xf), xf.astype(np.float64)
    off = np.zeros(B, np.int32) if offsets is None else np.asarray(offsets, np.int32)
    grok.grok_rope(x, None if offsets is None else U.dev(off))
    pos = off[:, None] + np.arange(T)[None, :]
    ref = orc.rope(x64, pos)
    if dtype == "bf16":
        U.assert_bf16_close(U.host(x), ref, "rope")
    else:
        U.assert_f32_close(U.host(x), ref, "rope")
    if offsets is None or 0 in list(off):
        b0 = int(np.argmax(off == 0))
        np.testing.assert_array_equal(U.host(x)[b0, 0], x64[b0, 0])  # position 0: identity


# --------------------------------------------------------------------------
# KV append
# --------------------------------------------------------------------------
def test_kv_append_rope_and_bit_exact_slots(G):
    grok, U, torch = G
    g = gi.rng(77)
    B, T, Tmax, Hq, Hkv, D = 3, 2, 64, 12, 2, 128
    kc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    kn, vn = gi.normal_bf16(g, (B, T, Hkv, D)), gi.normal_bf16(g, (B, T, Hkv, D))
    qb = gi.normal_bf16(g, (B, T, Hq, D))
    step = np.array([0, 30, 62], np.int32)
    kc, vc, q = U.dev_bf16(kc0), U.dev_bf16(vc0), U.dev_bf16(qb)
    new_step = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_kv_append(kc, vc, U.dev_bf16(kn), U.dev_bf16(vn), U.dev(step), q_inout=q,
                        new_step=new_step, status=status)
    torch.cuda.synchronize()
    assert status.item() == 0
    np.testing.assert_array_equal(new_step.cpu().numpy(), step + T)
    # reference rotation of the same values by the standalone RoPE entry point
    kr, qr = U.dev_bf16(kn), U.dev_bf16(qb)
    grok.grok_rope(kr, U.dev(step))
    grok.grok_rope(qr, U.dev(step))
    kcb, vcb = U.bits(kc), U.bits(vc)
    pos = step[:, None] + np.arange(T)[None]
    ref_k = orc.rope(orc.bf16_bits_to_f64(kn), pos)
    for b in range(B):
        sl = slice(step[b], step[b] + T)
        np.testing.assert_array_equal(vcb[b, sl], vn[b])             # V: bit copy
        np.testing.assert_array_equal(kcb[b, sl], U.bits(kr)[b])     # K: = grok_rope bits
        keep = np.ones(Tmax, bool)
        keep[sl] = False
        np.testing.assert_array_equal(kcb[b, keep], kc0[b, keep])    # other slots untouched
        np.testing.assert_array_equal(vcb[b, keep], vc0[b, keep])
    U.assert_bf16_close(orc.bf16_bits_to_f64(np.stack([kcb[b, step[b]:step[b] + T] for b in range(B)])),
                        ref_k, "roped k")
    np.testing.assert_array_equal(U.bits(q), U.bits(qr))
    U.assert_bf16_close(U.host(q), orc.rope(orc.bf16_bits_to_f64(qb), pos), "roped q")


def test_kv_append_out_of_range_and_no_rope(G):
    grok, U, torch = G
    g = gi.rng(78)
    B, T, Tmax, Hkv, D = 2, 2, 16, 1, 32
    kc0, vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D)), gi.normal_bf16(g, (B, Tmax, Hkv, D))
    kn, vn = gi.normal_bf16(g, (B, T, Hkv, D)), gi.normal_bf16(g, (B, T, Hkv, D))
    step = np.array([15, 4], np.int32)  # sequence 0 would overflow the cache
    kc, vc = U.dev_bf16(kc0), U.dev_bf16(vc0)
    ns = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_kv_append(kc, vc, U.dev_bf16(kn), U.dev_bf16(vn), U.dev(step), new_step=ns,
                        status=status, rope_base=0.0)
    torch.cuda.synchronize()
    assert status.item() == grok.GROK_ERANGE
    np.testing.assert_array_equal(ns.cpu().numpy(), [15, 6])
    kcb, vcb = U.bits(kc), U.bits(vc)
    np.testing.assert_array_equal(kcb[0], kc0[0])
    np.testing.assert_array_equal(vcb[0], vc0[0])
    np.testing.assert_array_equal(kcb[1, 4:6], kn[1])  # no RoPE: plain copy
    np.testing.assert_array_equal(vcb[1, 4:6], vn[1])


# --------------------------------------------------------------------------
# Prefill
# --------------------------------------------------------------------------
def _prefill_case(G, B, T, Hq, Hkv, D, dtype, mult, pad=None, kv_rows=None, seed=0):
    grok, U, torch = G
    p = gi.make_prefill_inputs(B, T, Hq, Hkv, D, seed=seed, dtype=dtype)
    to_dev = U.dev_bf16 if dtype == "bf16" else U.dev
    to64 = orc.bf16_bits_to_f64 if dtype == "bf16" else (lambda a: a.astype(np.float64))
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    if kv_rows is not None:  # K/V read in place from a longer buffer (cache stride)
        kk = torch.zeros((B, kv_rows, Hkv, D), dtype=q.dtype, device="cuda")
        vv = torch.zeros_like(kk)
        kk[:, :T] = k
        vv[:, :T] = v
        kk[:, T:] = 7.0  # finite garbage beyond T is never read
        vv[:, T:] = 7.0
        k, v = kk, vv
    kv = None if pad is None else U.dev(pad)
    out = torch.empty((B, T, Hq * D), dtype=q.dtype, device="cuda")
    grok.grok_attn_prefill(q, k, v, out, mult, 30.0, key_valid=kv)
    pos = np.broadcast_to(np.arange(T), (B, T))
    mask = orc.attention_mask(pos, T, key_valid=pad)
    ref = orc.attention(to64(p["q"]), to64(p["k"]), to64(p["v"]), mask, mult, 30.0)
    got = U.host(out)
    if dtype == "bf16":
        U.assert_bf16_close(got, ref, f"prefill B={B} T={T} Hq={Hq} Hkv={Hkv}")
    else:
        U.assert_f32_close(got, ref, f"prefill B={B} T={T}")
    return got, p


@pytest.mark.parametrize("B,T,Hq,Hkv,scale", [
    (2, 300, 48, 8, 4.0),   # Grok grouping, several query/key tiles, ragged tail
    (1, 64, 48, 8, 1.0),
    (1, 64, 8, 8, 1.0),     # MHA
    (1, 50, 12, 1, 1.0),    # one KV head, 12 query heads
    (1, 40, 16, 2, 2.0),    # 8 query heads per KV head
    (2, 33, 10, 2, 1.0),    # 5 per KV head
    (1, 1, 48, 8, 1.0),     # a single token
])
def test_prefill_mfma(G, B, T, Hq, Hkv, scale):
    _prefill_case(G, B, T, Hq, Hkv, 128, "bf16", scale / math.sqrt(128), seed=B * T + Hq)


@pytest.mark.parametrize("B,T,Hq,Hkv,Tmax,offsets", [
    (3, 37, 48, 8, 300, [0, 63, 263]),   # empty prefix, unaligned prefix, chunk ending at Tmax
    (2, 100, 6, 1, 256, [128, 5]),
    (1, 1, 16, 2, 64, [40]),             # one token: a decode step
    (2, 130, 12, 2, 400, [64, 270]),     # several query tiles
    (3, 70, 12, 2, 12400, [4100, 12330, 9]),  # long cached prefixes next to a short one
    (7, 20, 12, 2, 200, [150, 0, 75, 180, 3, 150, 90]),  # work ranking with a tie
    (65, 5, 6, 1, 48, [(7 * i) % 44 for i in range(65)]),  # more sequences than the ranking takes
    (2, 64, 48, 8, 4096, [0, 4032]),     # a 64-tile item next to a 1-tile one
    (3, 33, 12, 2, 3000, [991, 1024, 2967]),  # items of 16, 17 and 47 key tiles
    (1, 1, 16, 2, 4096, [4000]),         # one token, two head chunks, a long prefix
    (65, 5, 6, 1, 2200, [(34 * i) % 2196 for i in range(65)]),  # long prefixes without the ranking
])
def test_prefill_chunk(G, B, T, Hq, Hkv, Tmax, offsets):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    D, mult = 128, 1 / math.sqrt(128)
    p = gi.make_chunk_inputs(B, T, Hq, Hkv, D, Tmax, seed=B * T + Tmax, offsets=offsets)
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    st = pipe.ChunkStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                        U.dev(p["step"]), mult)
    out = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    np.testing.assert_array_equal(st.new_step.cpu().numpy(), np.asarray(offsets) + T)
    to64 = orc.bf16_bits_to_f64
    ref, kc2, vc2, _ = orc.chunk_prefill(to64(p["k_cache"]), to64(p["v_cache"]), to64(p["q"]), to64(p["k_new"]),
                                         to64(p["v_new"]), p["step"], mult)
    U.assert_bf16_close(out, ref, f"chunk B={B} T={T} offsets={offsets}")
    # the cache: v slots bit copies, k slots rotated, nothing else touched
    kcb, vcb = U.bits(kc), U.bits(vc)
    for b, o in enumerate(offsets):
        np.testing.assert_array_equal(vcb[b, o:o + T], p["v_new"][b])
        U.assert_bf16_close(to64(kcb[b, o:o + T]), kc2[b, o:o + T], "chunk k slots")
        np.testing.assert_array_equal(kcb[b, :o], p["k_cache"][b, :o])
        np.testing.assert_array_equal(kcb[b, o + T:], p["k_cache"][b, o + T:])


def test_prefill_chunk_at_offset_zero_is_the_prefill_bit_for_bit_and_bad_offsets(G):
    grok, U, torch = G
    B, T, Hq, Hkv, D, Tmax = 2, 150, 48, 8, 128, 256
    p = gi.make_chunk_inputs(B, T, Hq, Hkv, D, Tmax, seed=77, offsets=[0, 0])
    q, kc, vc = U.dev_bf16(p["q"]), U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    a = torch.empty((B, T, Hq * D), dtype=torch.bfloat16, device="cuda")
    b_ = torch.empty_like(a)
    grok.grok_attn_prefill_chunk(q, kc, vc, U.dev(p["step"]), a, 0.2)
    grok.grok_attn_prefill(q, kc, vc, b_, 0.2)          # K/V read in place, row stride Tmax
    np.testing.assert_array_equal(U.bits(a), U.bits(b_))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_attn_prefill_chunk(q, kc, vc, U.dev(np.array([-1, Tmax - T + 1], np.int32)), a, 0.2, status=status)
    torch.cuda.synchronize()
    assert status.item() == -34
    assert not np.any(U.host(a))


@pytest.mark.parametrize("B,T,Hq,Hkv,padded", [
    (1, 200, 48, 8, False),   # Grok-1 heads, a ragged last query tile
    (2, 129, 8, 8, False),    # MHA, two sequences
    (1, 64, 6, 1, False),     # MQA, one tile
    (2, 150, 12, 2, True),    # key padding (and a fully masked row in sequence 1)
])
def test_prefill_rope_matches_rope_then_prefill(G, B, T, Hq, Hkv, padded):
    """q rotated inside the attention kernel gives the bits of grok_rope(q)
    followed by grok_attn_prefill, and leaves q as it was."""
    grok, U, torch = G
    p = gi.make_prefill_inputs(B, T, Hq, Hkv, 128, seed=31 * T + Hq)
    q, k, v = U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"])
    grok.grok_rope(k, None, 1e4)
    kv = None
    if padded:
        g = gi.rng(7 + T)
        m = (g.uniform(size=(B, T)) > 0.3).astype(np.uint8)
        m[1, :] = 0
        m[1, T // 2:] = 1  # rows below T/2 of sequence 1 see no valid key
        kv = U.dev(m)
    mult = 1 / math.sqrt(128)
    ws = torch.empty(grok.grok_attn_prefill_rope_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    out_f = torch.empty((B, T, Hq * 128), dtype=torch.bfloat16, device="cuda")
    grok.grok_attn_prefill_rope(q, k, v, out_f, ws, mult, 30.0, key_valid=kv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(U.bits(q), p["q"])  # q untouched
    q2 = q.clone()
    grok.grok_rope(q2, None, 1e4)
    out_u = torch.empty_like(out_f)
    grok.grok_attn_prefill(q2, k, v, out_u, mult, 30.0, key_valid=kv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(U.bits(out_f), U.bits(out_u))


def test_prefill_mfma_padding_and_fully_masked_rows(G):
    B, T = 2, 77
    pad = np.ones((B, T), np.uint8)
    pad[0, :5] = 0          # rows 0..4 of sequence 0 see no valid key
    pad[0, 40:45] = 0
    pad[1, ::3] = 0
    U = G[1]
    got, p = _prefill_case(G, B, T, 48, 8, 128, "bf16", 1 / math.sqrt(128), pad=pad, seed=5)
    vmean = orc.bf16_bits_to_f64(p["v"])[0].mean(0)  # [Hkv, D] over all T keys
    for t in range(5):
        row = got[0, t].reshape(48, 128)
        for h in range(48):
            U.assert_bf16_close(row[h], vmean[h // 6], "fully masked row")


def test_prefill_mfma_cache_stride(G):
    _prefill_case(G, 2, 70, 48, 8, 128, "bf16", 1 / math.sqrt(128), kv_rows=100, seed=9)


def test_prefill_row0_equals_v0_bit_exact(G):
    grok, U, torch = G
    got, p = _prefill_case(G, 1, 96, 48, 8, 128, "bf16", 4 / math.sqrt(128), seed=11)
    v0 = orc.bf16_bits_to_f64(p["v"])[0, 0]  # [Hkv, D]
    for h in range(48):
        np.testing.assert_array_equal(got[0, 0, h * 128:(h + 1) * 128], v0[h // 6])


@pytest.mark.parametrize("B,T,Hq,Hkv,D,dtype,padded", [
    (1, 16, 6, 1, 32, "f32", False),
    (2, 45, 12, 2, 64, "bf16", True),
    (1, 20, 4, 2, 128, "f32", True),
    (1, 9, 3, 3, 256, "bf16", False),
])
def test_prefill_generic(G, B, T, Hq, Hkv, D, dtype, padded):
    pad = None
    if padded:
        pad = np.ones((B, T), np.uint8)
        pad[0, 0] = 0
        pad[-1, T // 2] = 0
    _prefill_case(G, B, T, Hq, Hkv, D, dtype, 1 / math.sqrt(D), pad=pad, seed=T + D)


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv,lens,Tmax", [
    (48, 8, [1, 127, 128, 129, 1024], 1024),
    (16, 1, [33, 300], 512),
    (8, 8, [5, 256], 256),
    (6, 3, [200, 77, 1], 200),  # capacity not a multiple of the 128-slot split
    (32, 16, [3, 500, 129], 640),  # two KV heads per die and sequence in the split layout
    (48, 8, [1, 900, 300, 1024, 129, 2, 640, 511, 777, 128, 1000], 1024),  # 11 sequences over 8 dies
    (8, 2, [100, 1, 513, 257, 64, 384, 200], 600),  # 14 (sequence, KV head) pairs: 2 empty die slots
])
def test_decode(G, Hq, Hkv, lens, Tmax):
    grok, U, torch = G
    B, D = len(lens), 128
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=Tmax + Hq, lengths=lens)
    kv_len = np.asarray(lens, np.int32)
    q = U.dev_bf16(p["q"])
    out = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8,
                     device="cuda")
    mult = 1 / math.sqrt(D)
    kc, vc, kl = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"]), U.dev(kv_len)
    grok.grok_attn_decode(q, kc, vc, kl, out, ws, mult)
    first = U.bits(out)
    # the arrival counters are left cleared: a second call on the same
    # workspace gives the same bits
    out.zero_()
    grok.grok_attn_decode(q, kc, vc, kl, out, ws, mult)
    np.testing.assert_array_equal(U.bits(out), first)
    mask = orc.attention_mask((kv_len - 1)[:, None], Tmax, kv_len=kv_len)
    ref = orc.attention(orc.bf16_bits_to_f64(p["q"]), orc.bf16_bits_to_f64(p["k_cache"]),
                        orc.bf16_bits_to_f64(p["v_cache"]), mask, mult, 30.0)
    U.assert_bf16_close(U.host(out), ref, "decode")
    assert U.rel_l2(U.host(out), ref) < 1e-2


@pytest.mark.parametrize("Hq,Hkv,lens,Tmax", [
    (48, 8, [300, 1, 129, 128], 300),   # a full cache, a one-slot sequence, split boundaries
    (6, 3, [200, 77, 1], 200),
    (16, 1, [1000], 1024),              # 16 query heads on one KV head
])
def test_decode_append_matches_unfused_calls(G, Hq, Hkv, lens, Tmax):
    """RoPE + append inside the split kernel give the bits of the append call
    followed by the decode call: output, both caches, rotated q, new_step."""
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    B, D = len(lens), 128
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=Hq * 7 + Tmax, lengths=lens)
    mult = 1 / math.sqrt(D)
    res = []
    for fused in (False, True):
        kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
        st = pipe.DecodeStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                             U.dev(p["step"]), mult, fused=fused)
        out = st()
        qo = torch.empty_like(st.q)
        if fused:  # the rotated q, as the unfused append leaves it in q
            grok.grok_attn_decode_append(st.q, st.k_new, st.v_new, kc, vc, st.step, out, st.workspace, mult,
                                         new_step=st.kv_len, q_out=qo, status=st.status)
        else:
            qo.copy_(st.q)
        torch.cuda.synchronize()
        assert st.status.item() == 0
        res.append((U.bits(out), U.bits(kc), U.bits(vc), U.bits(qo), st.kv_len.cpu().numpy()))
    for a, b_ in zip(*res):
        np.testing.assert_array_equal(a, b_)
    np.testing.assert_array_equal(res[1][4], lens)


def _poison_past(cache, lens):
    """NaN and Inf bit patterns in every cache slot at or past lens[b]."""
    c = cache.copy()
    for b, n in enumerate(lens):
        tail = c[b, n:]
        tail[...] = 0x7FC0                        # NaN
        tail[::2, ..., ::3] = 0x7F80              # +Inf
        tail[1::2, ..., 1::3] = 0xFF80            # -Inf
    return c


# 2 sequences: 16 (sequence, KV head) pairs x 8 splits, a grid resident at once
# (loads issued before the lengths arrive); 13 sequences: 832 workgroups, the
# lengths read first
@pytest.mark.parametrize("B", [2, 13])
def test_decode_reads_nothing_past_the_length(G, B):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    Hq, Hkv, D, Tmax = 48, 8, 128, 1024
    lens = [(397 * b + 129) % Tmax + 1 for b in range(B)]
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=41 + B, lengths=lens)
    mult = 1 / math.sqrt(D)
    kv_len = np.asarray(lens, np.int32)
    # decode against poisoned tails = decode against the clean cache, bit for bit
    outs = []
    for kcache, vcache in ((p["k_cache"], p["v_cache"]),
                           (_poison_past(p["k_cache"], lens), _poison_past(p["v_cache"], lens))):
        out = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8,
                         device="cuda")
        grok.grok_attn_decode(U.dev_bf16(p["q"]), U.dev_bf16(kcache), U.dev_bf16(vcache), U.dev(kv_len), out, ws,
                              mult)
        outs.append(U.bits(out))
    np.testing.assert_array_equal(outs[0], outs[1])
    mask = orc.attention_mask((kv_len - 1)[:, None], Tmax, kv_len=kv_len)
    ref = orc.attention(orc.bf16_bits_to_f64(p["q"]), orc.bf16_bits_to_f64(p["k_cache"]),
                        orc.bf16_bits_to_f64(p["v_cache"]), mask, mult, 30.0)
    U.assert_bf16_close(orc.bf16_bits_to_f64(outs[1]), ref, "decode, poisoned tails")
    # the fused step: slots past the new one poisoned
    res = []
    for poison in (False, True):
        kc0 = _poison_past(p["k_cache"], lens) if poison else p["k_cache"]
        vc0 = _poison_past(p["v_cache"], lens) if poison else p["v_cache"]
        kc, vc = U.dev_bf16(kc0), U.dev_bf16(vc0)
        st = pipe.DecodeStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                             U.dev(p["step"]), mult)
        out = st()
        torch.cuda.synchronize()
        assert st.status.item() == 0
        res.append(U.bits(out))
    np.testing.assert_array_equal(res[0], res[1])


def test_decode_grid_forms_agree(G):
    """A sequence decoded alone (a grid resident at once, loads issued before
    its length arrives) and within a batch of 13 (lengths read first) gives
    the same bits, plain and with the append."""
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    B, Hq, Hkv, D, Tmax = 13, 48, 8, 128, 1024
    lens = [(233 * b + 77) % Tmax + 1 for b in range(B)]
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=43, lengths=lens)
    mult = 1 / math.sqrt(D)

    def run(sl):
        n = sl.stop - sl.start
        kl = np.asarray(lens[sl], np.int32)
        out = torch.empty((n, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(grok.grok_attn_decode_workspace_bytes(n, Tmax, Hq, Hkv, D), dtype=torch.uint8,
                         device="cuda")
        grok.grok_attn_decode(U.dev_bf16(p["q"][sl]), U.dev_bf16(p["k_cache"][sl]), U.dev_bf16(p["v_cache"][sl]),
                              U.dev(kl), out, ws, mult)
        st = pipe.DecodeStep(U.dev_bf16(p["k_cache"][sl]), U.dev_bf16(p["v_cache"][sl]), U.dev_bf16(p["q"][sl]),
                             U.dev_bf16(p["k_new"][sl]), U.dev_bf16(p["v_new"][sl]), U.dev(p["step"][sl]), mult)
        fused = st()
        torch.cuda.synchronize()
        return U.bits(out), U.bits(fused), U.bits(st.k_cache), U.bits(st.v_cache)

    whole = run(slice(0, B))
    for b in (0, 5, 12):
        alone = run(slice(b, b + 1))
        for x, y in zip(whole, alone):
            np.testing.assert_array_equal(x[b:b + 1], y)


def test_decode_append_bad_step(G):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    B, Hq, Hkv, D, Tmax = 3, 12, 2, 128, 64
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=9, lengths=[10, 10, 10])
    steps = np.array([5, Tmax, -1], np.int32)
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    st = pipe.DecodeStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                         U.dev(steps), 0.1)
    out = U.host(st()).reshape(B, -1)
    torch.cuda.synchronize()
    assert st.status.item() == -34
    np.testing.assert_array_equal(st.kv_len.cpu().numpy(), [6, Tmax, -1])
    assert np.all(out[1:] == 0) and np.any(out[0] != 0)
    kcb = U.bits(kc)
    np.testing.assert_array_equal(kcb[1:], p["k_cache"][1:])   # nothing written for the bad ones
    np.testing.assert_array_equal(kcb[0, :5], p["k_cache"][0, :5])


def test_decode_bad_lengths_give_zero_rows_and_status(G):
    grok, U, torch = G
    B, Tmax, Hq, Hkv, D = 3, 256, 48, 8, 128
    p = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=3, lengths=[10, 10, 10])
    kv_len = np.array([0, 100, Tmax + 1], np.int32)
    out = torch.full((B, 1, Hq * D), 5.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8,
                     device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_attn_decode(U.dev_bf16(p["q"]), U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"]),
                          U.dev(kv_len), out, ws, 1 / math.sqrt(D), status=status)
    torch.cuda.synchronize()
    assert status.item() == grok.GROK_ERANGE
    got = U.host(out)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    mask = orc.attention_mask(np.array([[99]]), Tmax, kv_len=np.array([100]))
    ref = orc.attention(orc.bf16_bits_to_f64(p["q"][1:2]), orc.bf16_bits_to_f64(p["k_cache"][1:2]),
                        orc.bf16_bits_to_f64(p["v_cache"][1:2]), mask, 1 / math.sqrt(D))
    U.assert_bf16_close(got[1:2], ref, "valid row next to bad ones")


@pytest.mark.parametrize("B,d,Hq,Hkv,Tmax", [
    (1, 256, 4, 2, 300),
    (3, 1024, 8, 1, 64),      # x staged on chip (3 x 1024 values)
    (5, 256, 4, 2, 40),       # more rows than the on-chip path takes
    (20, 512, 16, 2, 33),     # two row tiles
])
def test_decode_qkv_matches_unfused_calls(G, B, d, Hq, Hkv, Tmax):
    """Projection + RoPE + cache write in one launch give the bits of the
    separate calls (few-row projection, then append with q in place)."""
    grok, U, torch = G
    D = 128
    g = gi.rng(B * 1000 + d)
    xb = gi.normal_bf16(g, (B, d))
    ws = [gi.int8_uniform(g, (d, n)) for n in (Hq * D, Hkv * D, Hkv * D)]
    ss = [(0.02 / 127 * g.uniform(0.5, 1.5, n)).astype(np.float32) for n in (Hq * D, Hkv * D, Hkv * D)]
    steps = g.integers(0, Tmax, size=B).astype(np.int32)
    steps[0] = Tmax - 1
    if B > 2:
        steps[1] = Tmax   # out of range: skipped
    kc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    x = U.dev_bf16(xb)
    wp = [grok.grok_linear_int8_pack(U.dev(w)) for w in ws]
    ds = [U.dev(s_) for s_ in ss]
    stp = U.dev(steps)
    # unfused
    q1 = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device="cuda")
    k1 = torch.empty((B, 1, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v1 = torch.empty_like(k1)
    kc1, vc1 = U.dev_bf16(kc0), U.dev_bf16(vc0)
    ns1 = torch.empty(B, dtype=torch.int32, device="cuda")
    st1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_linear_int8_gemv(x, wp, ds, [q1, k1, v1])
    grok.grok_kv_append(kc1, vc1, k1, v1, stp, q_inout=q1, new_step=ns1, status=st1)
    # fused
    q2 = torch.empty((B, Hq * D), dtype=torch.bfloat16, device="cuda")
    kc2, vc2 = U.dev_bf16(kc0), U.dev_bf16(vc0)
    ns2 = torch.empty(B, dtype=torch.int32, device="cuda")
    st2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    grok.grok_decode_qkv(x, wp[0], ds[0], wp[1], ds[1], wp[2], ds[2], q2, kc2, vc2, stp, new_step=ns2,
                         status=st2)
    torch.cuda.synchronize()
    ok = steps < Tmax
    # q: rotated where the append ran; where it was skipped, both hold the projection
    np.testing.assert_array_equal(U.bits(q2).reshape(B, Hq, D)[ok], U.bits(q1).reshape(B, Hq, D)[ok])
    np.testing.assert_array_equal(U.bits(kc2), U.bits(kc1))
    np.testing.assert_array_equal(U.bits(vc2), U.bits(vc1))
    np.testing.assert_array_equal(ns2.cpu().numpy(), ns1.cpu().numpy())
    assert st2.item() == st1.item() == (0 if ok.all() else -34)
    if not ok.all():
        np.testing.assert_array_equal(U.bits(q2).reshape(B, Hq, D)[~ok], U.bits(q1).reshape(B, Hq, D)[~ok])


@pytest.mark.parametrize("B,d,gamma", [(1, 6144, False), (2, 6144, True), (4, 1024, True)])
def test_decode_qkv_fused_norm(G, B, d, gamma):
    """With the pre-norm fused, against the oracle: norm, projections, RoPE at
    step[b], the cache slot written and no other."""
    grok, U, torch = G
    Hq, Hkv, D, Tmax = 4, 2, 128, 50
    g = gi.rng(B + d)
    xb = gi.normal_bf16(g, (B, d))
    gm = (g.uniform(0.5, 1.5, d)).astype(np.float32) if gamma else None
    ws = [gi.int8_uniform(g, (d, n)) for n in (Hq * D, Hkv * D, Hkv * D)]
    ss = [(0.02 / 127 * g.uniform(0.5, 1.5, n)).astype(np.float32) for n in (Hq * D, Hkv * D, Hkv * D)]
    steps = g.integers(0, Tmax, size=B).astype(np.int32)
    kc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D))
    wp = [grok.grok_linear_int8_pack(U.dev(w)) for w in ws]
    ds = [U.dev(s_) for s_ in ss]
    q = torch.empty((B, Hq * D), dtype=torch.bfloat16, device="cuda")
    kc, vc = U.dev_bf16(kc0), U.dev_bf16(vc0)
    grok.grok_decode_qkv(U.dev_bf16(xb), wp[0], ds[0], wp[1], ds[1], wp[2], ds[2], q, kc, vc, U.dev(steps),
                         prenorm=True, gamma=None if gm is None else U.dev(gm))
    x64 = orc.bf16_bits_to_f64(xb)
    n = orc.rmsnorm(x64, gm, 1e-5, out="bf16")
    pos = steps.reshape(B, 1).astype(np.int64)
    qr = orc.rope(orc.linear_int8(n, ws[0], ss[0], out="bf16").reshape(B, 1, Hq, D), pos)
    kr = orc.rope(orc.linear_int8(n, ws[1], ss[1], out="bf16").reshape(B, 1, Hkv, D), pos)
    vr = orc.linear_int8(n, ws[2], ss[2]).reshape(B, Hkv, D)
    U.assert_bf16_close(U.host(q).reshape(B, 1, Hq, D), qr, "fused q")
    kch, vch = U.host(kc), U.host(vc)
    for b in range(B):
        U.assert_bf16_close(kch[b, steps[b]], kr[b, 0], f"fused k slot b={b}")
        U.assert_bf16_close(vch[b, steps[b]], vr[b], f"fused v slot b={b}")
    mask = np.ones((B, Tmax), bool)
    mask[np.arange(B), steps] = False
    np.testing.assert_array_equal(U.bits(kc)[mask], kc0[mask])
    np.testing.assert_array_equal(U.bits(vc)[mask], vc0[mask])


# --------------------------------------------------------------------------
# Decode-time sub-layer (norm, few-row projections, RoPE + append, decode
# attention, output projection, post-norm + residual)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,d,Hq,Hkv,lens,Tmax,fused", [
    (3, 256, 4, 2, [300, 77, 1], 300, True),    # full, short and single-slot memories
    (3, 256, 4, 2, [300, 77, 1], 300, False),   # the same through separate calls
    (2, 1024, 16, 2, [129, 1000], 1024, True),  # 8 query heads per KV head
    (6, 256, 4, 2, [5, 6, 7, 8, 9, 10], 16, True),  # pre-norm not fused (more rows than on chip)
])
def test_decode_sublayer(G, B, d, Hq, Hkv, lens, Tmax, fused):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    D, mult = 128, 1 / math.sqrt(128)
    p = gi.make_decode_sublayer_inputs(B, d, Hq, Hkv, D, Tmax, seed=B * d + Tmax, lengths=lens,
                                       distinct_scales=True)
    dv = {k: (U.dev_bf16(v) if v.dtype == np.uint16 else U.dev(v)) for k, v in p.items()}
    st = pipe.DecodeSublayerStep(dv["x"], dv["k_cache"], dv["v_cache"], dv["step"], dv["wq"], dv["sq"],
                                 dv["wk"], dv["sk"], dv["wv"], dv["sv"], dv["wo"], dv["so"], Hq, Hkv, D,
                                 mult, fused=fused)
    y = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    np.testing.assert_array_equal(st.kv_len.cpu().numpy(), lens)
    x = orc.bf16_bits_to_f64(p["x"])
    kc, vc = orc.bf16_bits_to_f64(p["k_cache"]), orc.bf16_bits_to_f64(p["v_cache"])
    ref, kc2, vc2, _ = orc.decode_sublayer(x, kc, vc, p["step"], p["wq"], p["sq"], p["wk"], p["sk"],
                                           p["wv"], p["sv"], p["wo"], p["so"], Hq, Hkv, D, mult)
    # the appended slots (bf16 in both), then the output of the whole chain
    for b in range(B):
        s = lens[b] - 1
        U.assert_bf16_close(U.host(st.k_cache[b, s]), kc2[b, s], f"appended k b={b}")
        U.assert_bf16_close(U.host(st.v_cache[b, s]), vc2[b, s], f"appended v b={b}")
    nt = ref - x
    U.assert_bf16_close(y, ref, "decode sub-layer", magnitude=np.maximum(np.abs(ref), np.abs(nt)))


@pytest.mark.parametrize("B,d_in,d_out,use_gamma", [
    (1, 6144, 6144, False),   # one token at Grok-1's width: 384 workgroups meet through memory
    (3, 1024, 1000, True),    # a partial last 16-channel block, gamma
    (4, 8192, 512, True),     # the most rows of the widest input the fused form holds on chip
    (5, 256, 264, False),     # more rows: projection and norm as two launches
    (32, 1024, 2048, True),
])
def test_decode_out(G, B, d_in, d_out, use_gamma):
    """Output projection + post-norm + residual (one launch up to 4 rows)
    against the oracle's composition ([ch6] §6.3.1), against the separate
    projection + norm calls (at most one bf16 rounding apart), and bit-stable
    over repeated eager calls and graph replays (the arrival counter is
    reset by each call)."""
    grok, U, torch = G
    g = gi.rng(9000 + B * 7 + d_out)
    attn = gi.normal_bf16(g, (B, d_in))
    x = gi.normal_bf16(g, (B, d_out))
    w = gi.int8_uniform(g, (d_in, d_out))
    so = (0.02 / 127 * g.uniform(0.5, 1.5, d_out)).astype(np.float32)
    gm = g.uniform(0.5, 1.5, d_out).astype(np.float32) if use_gamma else None
    da, dx = U.dev_bf16(attn), U.dev_bf16(x)
    wp = grok.grok_linear_int8_pack(U.dev(w))
    dso = U.dev(so)
    dg = U.dev(gm) if use_gamma else None
    ws = torch.zeros(grok.grok_decode_out_workspace_bytes(B, d_in, d_out), dtype=torch.uint8, device="cuda")
    y = torch.empty((B, d_out), dtype=torch.bfloat16, device="cuda")
    grok.grok_decode_out(da, wp, dso, dx, y, ws, gamma=dg, eps=1e-5)
    torch.cuda.synchronize()
    y0 = U.bits(y).copy()
    a64, x64 = orc.bf16_bits_to_f64(attn), orc.bf16_bits_to_f64(x)
    o = orc.linear_int8(a64, w, so, out="bf16")
    ref = orc.rmsnorm(o, gm, 1e-5, residual=x64)
    nt = ref - x64
    U.assert_bf16_close(orc.bf16_bits_to_f64(y0), ref, f"decode_out B={B}", magnitude=np.maximum(np.abs(ref), np.abs(nt)))
    # the separate calls: the same o, the norm's sum in another order
    o_d = torch.empty((B, d_out), dtype=torch.bfloat16, device="cuda")
    y_u = torch.empty_like(y)
    grok.grok_linear_int8_gemv(da, [wp], [dso], [o_d])
    grok.grok_rmsnorm(o_d, y_u, gamma=dg, residual=dx, eps=1e-5)
    torch.cuda.synchronize()
    yu = orc.bf16_bits_to_f64(U.bits(y_u))
    yf = orc.bf16_bits_to_f64(y0)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(yu), 1e-30))[1] - 8)
    assert np.all(np.abs(yf - yu) <= ulp), "fused and separate calls differ by more than one bf16 rounding"
    assert np.mean(yf != yu) < 0.02
    # repeated calls, eager and from a graph, give the same bits
    for _ in range(2):
        grok.grok_decode_out(da, wp, dso, dx, y, ws, gamma=dg, eps=1e-5)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(U.bits(y), y0)
    gr = torch.cuda.CUDAGraph()
    y.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        grok.grok_decode_out(da, wp, dso, dx, y, ws, gamma=dg, eps=1e-5)
    for _ in range(3):
        y.zero_()
        gr.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(U.bits(y), y0)
    assert int(ws[:4].view(torch.int32).item()) == 0  # the counter is back at zero


# --------------------------------------------------------------------------
# MoE FFN sub-layer
# --------------------------------------------------------------------------
MOE_GATE_TOL = 1e-3


def _moe_dev(U, p):
    x = U.dev_bf16(p["x"])
    wr = U.dev(p["w_router"])
    experts = [tuple(U.dev(a) for a in ex) for ex in p["experts"]]
    return x, wr, experts


def _check_topk(probs, idx, k, tol=1e-5):
    """idx [T, k] is a valid choice of the k most probable experts: distinct,
    and none less probable than the k-th largest probability by more than tol
    (equal probabilities within rounding may be taken in either order)."""
    T, E = probs.shape
    assert idx.shape == (T, k)
    assert np.all((idx >= 0) & (idx < E))
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1]) if k > 1 else True
    kth = -np.sort(-probs, axis=1)[:, k - 1]
    chosen = np.take_along_axis(probs, idx.astype(np.int64), axis=1)
    assert np.all(chosen >= kth[:, None] - tol), np.max(kth[:, None] - chosen)
    # in probability order (slot 0 the most probable), up to ties
    assert np.all(chosen[:, :-1] >= chosen[:, 1:] - tol)


def test_moe_interleave(G):
    grok, U, torch = G
    g = gi.rng(77)
    d, F = 40, 24
    wg, wv = gi.int8_uniform(g, (d, F)), gi.int8_uniform(g, (d, F))
    sg, sv = g.uniform(0.5, 1.5, F).astype(np.float32), g.uniform(0.5, 1.5, F).astype(np.float32)
    wgv, sgv = grok.grok_moe_interleave(U.dev(wg), U.dev(sg), U.dev(wv), U.dev(sv))
    torch.cuda.synchronize()
    ref = np.empty((d, 2 * F), np.int8)
    refs = np.empty(2 * F, np.float32)
    for q in range(F // 4):
        ref[:, 8 * q:8 * q + 4], ref[:, 8 * q + 4:8 * q + 8] = wg[:, 4 * q:4 * q + 4], wv[:, 4 * q:4 * q + 4]
        refs[8 * q:8 * q + 4], refs[8 * q + 4:8 * q + 8] = sg[4 * q:4 * q + 4], sv[4 * q:4 * q + 4]
    assert np.array_equal(wgv.cpu().numpy(), ref)
    assert np.array_equal(sgv.cpu().numpy(), refs)


@pytest.mark.parametrize("T,d,E,k", [(37, 6144, 8, 2), (1, 64, 3, 2), (300, 200, 8, 4), (9, 8, 1, 1)])
def test_moe_route(G, T, d, E, k):
    grok, U, torch = G
    g = gi.rng(T + d)
    nb = gi.normal_bf16(g, (T, d))
    wr = (gi.normal_f32(g, (d, E)) * np.float32(1.5 / math.sqrt(d))).astype(np.float32)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
    grok.grok_moe_route(U.dev_bf16(nb), U.dev(wr), idx, gates)
    torch.cuda.synchronize()
    probs, _, _ = orc.moe_route(orc.bf16_bits_to_f64(nb), wr, k)
    gi_ = idx.cpu().numpy()
    _check_topk(probs, gi_, k)
    U.assert_f32_close(gates.cpu().numpy(), np.take_along_axis(probs, gi_.astype(np.int64), axis=1), "gates")


def _skewed_router(g, d, E, x_bits):
    """Router weights under which most rows pick expert 0 first and none picks
    expert E-1: both columns follow a direction u that every row of x shares."""
    x = orc.bf16_bits_to_f64(x_bits)
    u = np.sign(g.standard_normal(d))
    x = x + u                                          # every row leans along u
    wr = (gi.normal_f32(g, (d, E)) * np.float32(1.5 / math.sqrt(d))).astype(np.float32)
    wr[:, 0] += (u * 5.0 / d).astype(np.float32)       # logit about +3.5 for expert 0
    wr[:, E - 1] -= (u * 20.0 / d).astype(np.float32)  # about -14 for expert E-1
    return gi.f32_to_bf16_bits(x.astype(np.float32)), wr


@pytest.mark.parametrize("T,d,F,E,k,case", [
    (600, 256, 384, 4, 2, "plain"),      # ~300 rows per expert: two row tiles, ragged
    (333, 200, 72, 8, 2, "distinct"),    # K and N tails in both products, per-channel scales
    (1, 64, 32, 8, 2, "plain"),          # a single token
    (130, 128, 64, 3, 2, "plain"),       # three experts
    (200, 64, 48, 4, 4, "distinct"),     # every expert chosen by every token
    (520, 128, 96, 8, 2, "skewed"),      # one large group, one empty expert
])
def test_moe_ffn(G, T, d, F, E, k, case):
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    p = gi.make_moe_inputs(1, T, d, F, E, seed=900 + T, distinct_scales=(case == "distinct"),
                           scale_up=1.0 / (127 * math.sqrt(d) * 0.58), scale_down=1.0 / (127 * math.sqrt(F) * 0.58 * 0.4))
    p["x"] = p["x"].reshape(T, d)
    if case == "skewed":
        p["x"], p["w_router"] = _skewed_router(gi.rng(5), d, E, p["x"])
    x, wr, experts = _moe_dev(U, p)
    step = pipe.MoeStep(x, wr, experts, k=k)
    y = step()
    torch.cuda.synchronize()
    idx = step.idx.cpu().numpy().astype(np.int64)
    x64 = orc.bf16_bits_to_f64(p["x"])
    n = orc.rmsnorm(x64, None, 1e-5, out="bf16")
    probs, _, _ = orc.moe_route(n, p["w_router"], k)
    # The router's own arithmetic is checked on identical inputs above; here its
    # input is the GPU's normalised rows, which may differ from the oracle's by
    # one bf16 rounding in a few elements (fp32 vs fp64 norm), moving a logit
    # by up to about |w_r| * 2^-8: the probabilities get a looser bound.
    _check_topk(probs, idx, k, tol=MOE_GATE_TOL)
    gerr = np.abs(step.gates.cpu().numpy() - np.take_along_axis(probs, idx, axis=1)).max()
    assert gerr <= MOE_GATE_TOL, gerr
    if case == "skewed":
        counts = np.bincount(idx.ravel(), minlength=E)
        assert counts[0] > T // 2 and counts[E - 1] == 0, counts
    ref, _, _ = orc.moe_sublayer(x64, p["w_router"], p["experts"], 1e-5, k, idx=idx)
    # y = x + n(mix): the relative part of the bound belongs to the larger of |y|
    # and the normalised summand, here ref - x (exact up to ref's rounding)
    nm = ref - x64
    assert np.abs(U.host(y) - x64).max() > 0.5  # the expert branch contributed
    err = U.assert_bf16_close(U.host(y), ref, f"moe {case}", magnitude=np.maximum(np.abs(ref), np.abs(nm)))
    print(f"moe T={T} d={d} F={F} E={E} k={k} {case}: max abs err {err:.2e}, rel L2 {U.rel_l2(U.host(y), ref):.2e}")


def test_moe_ffn_repeat_and_empty(G):
    """Two calls on the same buffers give the same bits (the plan is rebuilt
    every call, nothing carries over); T = 0 is a no-op."""
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    p = gi.make_moe_inputs(1, 100, 128, 64, 8, seed=31)
    x, wr, experts = _moe_dev(U, p)
    step = pipe.MoeStep(x.reshape(100, 128), wr, experts)
    a = U.bits(step()).copy()
    b = U.bits(step())
    assert np.array_equal(a, b)
    e = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    grok.grok_moe_ffn(e, wr, step.wgv, step.sgv, step.w1, step.s1, torch.empty_like(e), ws)


def test_slot_insertion_into_a_batched_cache_then_batched_decode(G):
    """Continuous batching through the C ABI: a new prompt is prefilled into one
    free slot of a batched cache (append + chunk attention on that slot's view,
    offset 0), leaving the other slots' bytes untouched; then one batched decode
    step runs over every slot at its own position. The inserted slot's prefill
    equals the cache-free prefill bit for bit, and every decode row matches the
    oracle's decode step of that sequence."""
    grok, U, torch = G
    g = gi.rng(91)
    B, Tmax, Hq, Hkv, D, T = 4, 256, 12, 2, 128, 100
    mult, slot = 0.2, 2
    kc0, vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D)), gi.normal_bf16(g, (B, Tmax, Hkv, D))
    kc, vc = U.dev_bf16(kc0), U.dev_bf16(vc0)
    qp, kp, vp = gi.normal_bf16(g, (1, T, Hq, D)), gi.normal_bf16(g, (1, T, Hkv, D)), gi.normal_bf16(g, (1, T, Hkv, D))
    q = U.dev_bf16(qp)
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ks, vs = kc[slot:slot + 1], vc[slot:slot + 1]          # views of one slot (batch-major: contiguous)
    grok.grok_kv_append(ks, vs, U.dev_bf16(kp), U.dev_bf16(vp), zero, q_inout=q, status=status)
    out = torch.empty((1, T, Hq * D), dtype=torch.bfloat16, device="cuda")
    grok.grok_attn_prefill_chunk(q, ks, vs, zero, out, mult, status=status)
    # the same prompt without a cache: RoPE q and k at 0..T-1, causal prefill
    qr, kr = U.dev_bf16(qp), U.dev_bf16(kp)
    grok.grok_rope(qr)
    grok.grok_rope(kr)
    ref = torch.empty_like(out)
    grok.grok_attn_prefill(qr, kr, U.dev_bf16(vp), ref, mult)
    torch.cuda.synchronize()
    assert status.item() == 0
    np.testing.assert_array_equal(U.bits(out), U.bits(ref))
    kcb, vcb = U.bits(kc), U.bits(vc)
    for b in range(B):
        if b != slot:
            np.testing.assert_array_equal(kcb[b], kc0[b])
            np.testing.assert_array_equal(vcb[b], vc0[b])
    np.testing.assert_array_equal(kcb[slot, T:], kc0[slot, T:])
    np.testing.assert_array_equal(kcb[slot, :T], U.bits(kr)[0])
    # one batched decode step: every slot continues at its own position
    step = np.array([50, 120, T, 30], np.int32)
    qn, kn, vn = (gi.normal_bf16(g, (B, 1, Hq, D)), gi.normal_bf16(g, (B, 1, Hkv, D)),
                  gi.normal_bf16(g, (B, 1, Hkv, D)))
    dout = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8, device="cuda")
    kc_before, vc_before = orc.bf16_bits_to_f64(U.bits(kc)), orc.bf16_bits_to_f64(U.bits(vc))
    grok.grok_attn_decode_append(U.dev_bf16(qn), U.dev_bf16(kn), U.dev_bf16(vn), kc, vc, U.dev(step), dout, ws,
                                 mult, status=status)
    torch.cuda.synchronize()
    assert status.item() == 0
    ref_out, _, _, _ = orc.decode_step(kc_before, vc_before, orc.bf16_bits_to_f64(qn), orc.bf16_bits_to_f64(kn),
                                       orc.bf16_bits_to_f64(vn), step, mult)
    U.assert_bf16_close(U.host(dout), ref_out, "batched decode after slot insertion")


# --------------------------------------------------------------------------
# Fused Q/K/V projection with RoPE and the cache write (prefill)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,d,Hq,Hkv,Tmax,steps", [
    (2, 300, 256, 6, 2, 512, [0, 137]),     # ragged row tiles, two positions
    (1, 77, 200, 4, 1, 77, None),           # step NULL: the cache is the prompt's K/V; K tail
    (3, 64, 6144, 48, 8, 128, [64, 0, 10]),  # Grok-1 widths
])
def test_prefill_qkv_matches_projections_then_append(G, B, T, d, Hq, Hkv, Tmax, steps):
    """Bit-identical to three grok_linear_int8 calls and grok_kv_append (which
    rotates q and k with the same pinned arithmetic), and within tolerance of
    the oracle's rope(x W) at the same positions; cache slots outside
    [step, step + T) are untouched."""
    grok, U, torch = G
    g = gi.rng(d + T)
    D = 128
    xb = gi.normal_bf16(g, (B, T, d))
    ws = {n: gi.int8_uniform(g, (d, h * D)) for n, h in (("q", Hq), ("k", Hkv), ("v", Hkv))}
    sc = {n: (g.uniform(0.5, 1.5, w.shape[1]) / (127 * math.sqrt(d) * 0.58)).astype(np.float32)
          for n, w in ws.items()}
    kc0, vc0 = gi.normal_bf16(g, (B, Tmax, Hkv, D)), gi.normal_bf16(g, (B, Tmax, Hkv, D))
    x = U.dev_bf16(xb)
    W = {n: U.dev(w) for n, w in ws.items()}
    S = {n: U.dev(s) for n, s in sc.items()}
    st = None if steps is None else U.dev(np.array(steps, np.int32))
    q = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc, vc = U.dev_bf16(kc0), U.dev_bf16(vc0)
    new_step = torch.zeros(B, dtype=torch.int32, device="cuda") if steps is not None else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(grok.grok_prefill_qkv_workspace_bytes(Tmax), dtype=torch.uint8, device="cuda")
    grok.grok_prefill_qkv(x, W["q"], S["q"], W["k"], S["k"], W["v"], S["v"], q, kc, vc, wsp, step=st,
                          new_step=new_step, status=status)
    # unfused: three projections, then append (RoPE of q in place and of k into the cache)
    q2 = torch.empty_like(q)
    k2 = torch.empty((B, T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    v2 = torch.empty_like(k2)
    for out, n in ((q2, "q"), (k2, "k"), (v2, "v")):
        grok.grok_linear_int8(x, W[n], S[n], out)
    kc2, vc2 = U.dev_bf16(kc0), U.dev_bf16(vc0)
    st2 = st if st is not None else torch.zeros(B, dtype=torch.int32, device="cuda")
    grok.grok_kv_append(kc2, vc2, k2, v2, st2, q_inout=q2)
    torch.cuda.synchronize()
    assert status.item() == 0
    np.testing.assert_array_equal(U.bits(q), U.bits(q2))
    np.testing.assert_array_equal(U.bits(kc), U.bits(kc2))
    np.testing.assert_array_equal(U.bits(vc), U.bits(vc2))
    s0 = np.zeros(B, np.int64) if steps is None else np.array(steps)
    if new_step is not None:
        np.testing.assert_array_equal(new_step.cpu().numpy(), s0 + T)
    kcb = U.bits(kc)
    for b in range(B):
        keep = np.ones(Tmax, bool)
        keep[s0[b]:s0[b] + T] = False
        np.testing.assert_array_equal(kcb[b, keep], kc0[b, keep])
    # oracle on a few rows
    x64 = orc.bf16_bits_to_f64(xb)
    for b in range(B):
        rows = np.array([0, T - 1, T // 2])
        pos = (s0[b] + rows)[None]
        qr = orc.rope(orc.linear_int8(x64[b, rows], ws["q"], sc["q"], out="bf16").reshape(1, len(rows), Hq, D), pos)
        kr = orc.rope(orc.linear_int8(x64[b, rows], ws["k"], sc["k"], out="bf16").reshape(1, len(rows), Hkv, D), pos)
        U.assert_bf16_close(U.host(q[b, rows])[None], qr, f"fused q b={b}")
        U.assert_bf16_close(orc.bf16_bits_to_f64(kcb[b, s0[b] + rows])[None], kr, f"fused k b={b}")


def test_prefill_qkv_out_of_range_sequence_writes_nothing(G):
    grok, U, torch = G
    g = gi.rng(5)
    B, T, d, Hq, Hkv, Tmax, D = 2, 40, 64, 2, 1, 64, 128
    x = U.dev_bf16(gi.normal_bf16(g, (B, T, d)))
    w = {n: U.dev(gi.int8_uniform(g, (d, h * D))) for n, h in (("q", Hq), ("k", Hkv), ("v", Hkv))}
    s = {n: torch.full((t.shape[1],), 1e-3, dtype=torch.float32, device="cuda") for n, t in w.items()}
    q = torch.zeros((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Tmax, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    step = U.dev(np.array([30, 10], np.int32))   # sequence 0: 30 + 40 > 64
    new_step = torch.zeros(B, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsp = torch.empty(grok.grok_prefill_qkv_workspace_bytes(Tmax), dtype=torch.uint8, device="cuda")
    grok.grok_prefill_qkv(x, w["q"], s["q"], w["k"], s["k"], w["v"], s["v"], q, kc, vc, wsp, step=step,
                          new_step=new_step, status=status)
    torch.cuda.synchronize()
    assert status.item() == -34
    np.testing.assert_array_equal(new_step.cpu().numpy(), [30, 50])
    assert not U.host(q[0]).any() and not U.host(kc[0]).any() and not U.host(vc[0]).any()
    assert U.host(q[1]).any() and U.host(kc[1, 10:50]).any() and not U.host(kc[1, 50:]).any()


def test_sublayer_fused_front_half_is_bit_identical(G):
    """The sub-layer with the fused Q/K/V launch gives the bits of the one with
    separate projections and RoPE passes."""
    grok, U, torch = G
    import gqa_attention_grok_amd.pipeline as pipe
    p = gi.make_sublayer_inputs(1, 300, 1024, 8, 2, 128, seed=12)
    dv = {k: (U.dev_bf16(v) if k == "x" else U.dev(v)) for k, v in p.items()}
    outs = []
    for fused in (True, False):
        st = pipe.SublayerStep(dv["x"], dv["wq"], dv["sq"], dv["wk"], dv["sk"], dv["wv"], dv["sv"], dv["wo"],
                               dv["so"], 8, 2, 128, 1 / math.sqrt(128), fused=fused)
        outs.append(U.bits(st()).copy())
    np.testing.assert_array_equal(outs[0], outs[1])
