"""The named workloads at full size, run through the same step objects the
benchmark times, checked against the fp64 oracle: in full where the oracle is
cheap (tiny prefill, both decodes, the one-sequence decode sub-layer), on
sampled output rows or sequences that the oracle computes one by one otherwise
(8k prefill, full sub-layer, ragged decode sub-layer)."""
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
    import gqa_attention_grok_amd.pipeline as pipe
    import gpu_util
    return grok, pipe, gpu_util, torch


def test_prefill_f32_t16(G):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["prefill_f32_t16"]
    p = gi.make_workload(w.name)
    step = pipe.PrefillStep(U.dev(p["q"]), U.dev(p["k"]), U.dev(p["v"]), w.attn_mult, w.softcap)
    out = U.host(step())
    pos = np.arange(w.T)[None]
    q = orc.rope(p["q"].astype(np.float64), pos, out="f32")
    k = orc.rope(p["k"].astype(np.float64), pos, out="f32")
    ref = orc.attention(q, k, p["v"].astype(np.float64), orc.attention_mask(pos, w.T), w.attn_mult,
                        w.softcap)
    err = U.assert_f32_close(out, ref, "tiny prefill")
    print(f"tiny prefill max abs err {err:.2e}")


def _decode_check(G, name):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS[name]
    p = gi.make_workload(name)
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    step = pipe.DecodeStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                           U.dev(p["step"]), w.attn_mult, w.softcap)
    out = U.host(step())
    torch.cuda.synchronize()
    assert step.status.item() == 0
    np.testing.assert_array_equal(step.kv_len.cpu().numpy(), p["kv_len"])
    B = w.B
    # oracle: RoPE q and k_new at step[b], append, attend [0, step+1)
    q = orc.bf16_bits_to_f64(p["q"])
    kn = orc.bf16_bits_to_f64(p["k_new"])
    vn = orc.bf16_bits_to_f64(p["v_new"])
    pos = p["step"].reshape(B, 1)
    qr = orc.rope(q, pos, out="bf16")
    kr = orc.rope(kn, pos, out="bf16")
    kr_exact = orc.rope(kn, pos)
    kcb, vcb = U.bits(kc), U.bits(vc)
    errs = []
    for b in range(B):
        s = int(p["step"][b])
        # cache: V slot bit copy, K slot roped, every other slot untouched
        np.testing.assert_array_equal(vcb[b, s], p["v_new"][b, 0])
        U.assert_bf16_close(orc.bf16_bits_to_f64(kcb[b, s]), kr_exact[b, 0], "appended k")
        np.testing.assert_array_equal(kcb[b, :s], p["k_cache"][b, :s])
        np.testing.assert_array_equal(kcb[b, s + 1:], p["k_cache"][b, s + 1:])
        np.testing.assert_array_equal(vcb[b, :s], p["v_cache"][b, :s])
        np.testing.assert_array_equal(vcb[b, s + 1:], p["v_cache"][b, s + 1:])
        L = s + 1
        k64 = orc.bf16_bits_to_f64(p["k_cache"][b:b + 1, :L])
        v64 = orc.bf16_bits_to_f64(p["v_cache"][b:b + 1, :L])
        k64[0, s] = kr[b, 0]
        v64[0, s] = vn[b, 0]
        ref = orc.attention(qr[b:b + 1], k64, v64, np.ones((1, 1, L), bool), w.attn_mult, w.softcap)
        errs.append(U.assert_bf16_close(out[b:b + 1], ref, f"{name} b={b}"))
        # stricter self-check: the outputs are small averages, so also bound the
        # error relative to the output scale
        assert np.max(np.abs(out[b:b + 1] - ref)) <= 2e-2 * np.max(np.abs(ref))
        assert U.rel_l2(out[b:b + 1], ref) < 1e-2
    print(f"{name} max abs err {max(errs):.2e}")


def test_decode_b1_t8192(G):
    _decode_check(G, "decode_b1_t8192")


def test_decode_ragged_b32_t8192(G):
    _decode_check(G, "decode_ragged_b32_t8192")


def test_prefill_b1_t8192_sampled(G):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["prefill_b1_t8192"]
    p = gi.make_workload(w.name)
    step = pipe.PrefillStep(U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"]), w.attn_mult,
                            w.softcap)
    out = step()
    torch.cuda.synchronize()
    T, Hq, Hkv, D = w.T, w.Hq, w.Hkv, w.D
    pos = np.arange(T)[None]
    k = orc.rope(orc.bf16_bits_to_f64(p["k"]), pos, out="bf16")
    v = orc.bf16_bits_to_f64(p["v"])
    g = gi.rng(31337)
    rows = [0, 1, 31, 32, 4095, 8190, 8191] + list(g.integers(0, T, 25))
    got = U.host(out[0, rows]).reshape(len(rows), Hq, D)
    # row 0 attends only to key 0: its weight is exactly one
    for h in range(Hq):
        np.testing.assert_array_equal(got[0, h], v[0, 0, h // (Hq // Hkv)])
    errs = []
    for r, t in enumerate(rows):
        qt = orc.rope(orc.bf16_bits_to_f64(p["q"][:, t:t + 1]), np.array([[t]]), out="bf16")
        mask_row = np.arange(T) <= t
        for h in range(Hq):
            ref = orc.attention_rows(qt, k, v, 0, 0, h, mask_row, w.attn_mult, w.softcap)
            errs.append(U.assert_bf16_close(got[r, h], ref, f"prefill t={t} h={h}"))
    print(f"prefill sampled {len(rows)} rows x {Hq} heads, max abs err {max(errs):.2e}")


def test_prefill_padded_b2_t4096_sampled(G):
    """Long prompts with key padding (10 % of the keys, and the whole first 64
    keys of sequence 1): sampled rows of every head against the oracle, the
    first rows of sequence 1 having no valid key at all (equal weights over
    all T value rows)."""
    grok, pipe, U, torch = G
    B, T, Hq, Hkv, D = 2, 4096, 48, 8, 128
    mult = 1 / np.sqrt(D)
    p = gi.make_prefill_inputs(B, T, Hq, Hkv, D, seed=2024, key_pad_frac=0.1)
    kv = p["key_valid"].copy()
    kv[1, :64] = 0
    out = torch.empty((B, T, Hq * D), dtype=torch.bfloat16, device="cuda")
    grok.grok_attn_prefill(U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"]), out, mult,
                           key_valid=U.dev(kv))
    torch.cuda.synchronize()
    q, k, v = (orc.bf16_bits_to_f64(p[n]) for n in ("q", "k", "v"))
    g = gi.rng(4242)
    rows = [0, 1, 63, 64, 65, 2047, 4094, 4095] + list(g.integers(0, T, 8))
    for b in range(B):
        got = U.host(out[b, rows]).reshape(len(rows), Hq, D)
        for r, t in enumerate(rows):
            mask_row = (np.arange(T) <= t) & (kv[b] != 0)
            for h in range(Hq):
                ref = orc.attention_rows(q, k, v, b, t, h, mask_row, mult)
                U.assert_bf16_close(got[r, h], ref, f"padded prefill b={b} t={t} h={h}")


def test_prefill_b1_t8192_two_heads_every_row(G):
    """Every one of the 8192 query rows of two heads in different KV groups
    (head 0 on KV head 0, head 47 on KV head 7) against the oracle: all 256
    query tiles of the 8k prefill, at the launch the benchmark times."""
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["prefill_b1_t8192"]
    p = gi.make_workload(w.name)
    step = pipe.PrefillStep(U.dev_bf16(p["q"]), U.dev_bf16(p["k"]), U.dev_bf16(p["v"]), w.attn_mult,
                            w.softcap)
    out = step()
    torch.cuda.synchronize()
    T, Hq, Hkv, D = w.T, w.Hq, w.Hkv, w.D
    G_ = Hq // Hkv
    pos = np.arange(T)[None]
    k = orc.rope(orc.bf16_bits_to_f64(p["k"]), pos, out="bf16")
    v = orc.bf16_bits_to_f64(p["v"])
    errs = []
    for h in (0, Hq - 1):
        g = h // G_
        got = U.host(out[0, :, h * D:(h + 1) * D])
        qh = orc.rope(orc.bf16_bits_to_f64(p["q"][:, :, h:h + 1]), pos, out="bf16")
        for r0 in range(0, T, 512):
            rows = np.arange(r0, r0 + 512)[None]
            ref = orc.attention(qh[:, r0:r0 + 512], k[:, :, g:g + 1], v[:, :, g:g + 1],
                                orc.attention_mask(rows, T), w.attn_mult, w.softcap)[0]
            errs.append(U.assert_bf16_close(got[r0:r0 + 512], ref, f"prefill h={h} rows {r0}..{r0 + 511}"))
    print(f"prefill 2 heads x {T} rows, max abs err {max(errs):.2e}")


def test_sublayer_b4_t2048_sampled(G):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["sublayer_b4_t2048"]
    p = gi.make_workload(w.name)
    dv = {k: (U.dev_bf16(v) if k == "x" else U.dev(v)) for k, v in p.items()}
    step = pipe.SublayerStep(dv["x"], dv["wq"], dv["sq"], dv["wk"], dv["sk"], dv["wv"], dv["sv"],
                             dv["wo"], dv["so"], w.Hq, w.Hkv, w.D, w.attn_mult, w.softcap, w.eps)
    y = step()
    torch.cuda.synchronize()
    B, T, d, Hq, Hkv, D = w.B, w.T, w.d_model, w.Hq, w.Hkv, w.D
    x = orc.bf16_bits_to_f64(p["x"])
    n = orc.rmsnorm(x, None, w.eps, out="bf16")
    U.assert_bf16_close(U.host(step.n), orc.rmsnorm(x, None, w.eps), "sublayer pre-norm")
    g = gi.rng(4242)
    errs = []
    for b in (0, 3):
        kb = orc.linear_int8(n[b], p["wk"], p["sk"], out="bf16").reshape(1, T, Hkv, D)
        vb = orc.linear_int8(n[b], p["wv"], p["sv"]).reshape(1, T, Hkv, D)
        U.assert_bf16_close(U.host(step.v[b:b + 1]), vb, "sublayer v projection")
        vb = orc.round_bf16(vb)
        U.assert_bf16_close(U.host(step.k[b:b + 1]), orc.rope(kb, np.arange(T)[None]), "sublayer roped k")
        kb = orc.rope(kb, np.arange(T)[None], out="bf16")
        for t in [0, 1, 2047] + list(g.integers(0, T, 5)):
            qt = orc.linear_int8(n[b, t], p["wq"], p["sq"], out="bf16").reshape(1, 1, Hq, D)
            qt = orc.rope(qt, np.array([[t]]), out="bf16")
            mask_row = np.arange(T) <= t
            a = np.concatenate([orc.attention_rows(qt, kb, vb, 0, 0, h, mask_row, w.attn_mult, w.softcap)
                                for h in range(Hq)])
            ga = U.host(step.attn[b, t])
            U.assert_bf16_close(ga, a, f"sublayer attention b={b} t={t}")
            a = orc.round_bf16(a)
            o = orc.linear_int8(a, p["wo"], p["so"])
            go = U.host(step.o[b, t])
            print(f"sublayer b={b} t={t}: rel L2 attention {U.rel_l2(ga, a):.2e}, "
                  f"out-proj {U.rel_l2(go, o):.2e}", flush=True)
            U.assert_bf16_close(go, o, f"sublayer output projection b={b} t={t}")
            o = orc.round_bf16(o)
            # post-norm handed on in bf16, then the residual add (exact; the GPU rounds it)
            nt = orc.rmsnorm(o[None], None, w.eps, out="bf16")[0]
            yt = x[b, t] + nt
            # The residual add is exact up to its last rounding, so the relative
            # part of the bound applies to the larger of |y| and the normalised
            # summand |n|: when x and n nearly cancel, |y| is small while n
            # carries its own bf16 error at its own magnitude.
            errs.append(U.assert_bf16_close(U.host(y[b, t]), yt, f"sublayer output b={b} t={t}",
                                            magnitude=np.maximum(np.abs(yt), np.abs(nt))))
    print(f"sublayer sampled rows, max abs err {max(errs):.2e}")


@pytest.mark.parametrize("name,seqs", [
    ("decode_sublayer_b1_t8192", None),
    ("decode_sublayer_b32_t8192", (0, 13, 31)),
])
def test_decode_sublayer_workloads(G, name, seqs):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS[name]
    p = gi.make_workload(name)
    dv = {k: (U.dev_bf16(v) if v.dtype == np.uint16 else U.dev(v)) for k, v in p.items()}
    st = pipe.DecodeSublayerStep(dv["x"], dv["k_cache"], dv["v_cache"], dv["step"], dv["wq"], dv["sq"],
                                 dv["wk"], dv["sk"], dv["wv"], dv["sv"], dv["wo"], dv["so"], w.Hq, w.Hkv,
                                 w.D, w.attn_mult, w.softcap, w.eps)
    y = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    np.testing.assert_array_equal(st.kv_len.cpu().numpy(), p["kv_len"])
    del dv
    seqs = range(w.B) if seqs is None else seqs
    errs = []
    for b in seqs:  # sequences are independent: the oracle takes them one at a time
        sl = slice(b, b + 1)
        x = orc.bf16_bits_to_f64(p["x"][sl])
        ref, _, _, _ = orc.decode_sublayer(
            x, orc.bf16_bits_to_f64(p["k_cache"][sl]), orc.bf16_bits_to_f64(p["v_cache"][sl]),
            p["step"][sl], p["wq"], p["sq"], p["wk"], p["sk"], p["wv"], p["sv"], p["wo"], p["so"],
            w.Hq, w.Hkv, w.D, w.attn_mult, w.softcap, w.eps)
        nt = ref - x
        errs.append(U.assert_bf16_close(y[sl], ref, f"{name} b={b} (length {p['kv_len'][b]})",
                                        magnitude=np.maximum(np.abs(ref), np.abs(nt))))
        print(f"{name} b={b}: rel L2 {U.rel_l2(y[sl], ref):.2e}", flush=True)
    print(f"{name}: max abs err {max(errs):.2e}")


def test_prefill_chunk_b4_t512_sampled(G):
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["prefill_chunk_b4_t512"]
    p = gi.make_workload(w.name)
    kc, vc = U.dev_bf16(p["k_cache"]), U.dev_bf16(p["v_cache"])
    st = pipe.ChunkStep(kc, vc, U.dev_bf16(p["q"]), U.dev_bf16(p["k_new"]), U.dev_bf16(p["v_new"]),
                        U.dev(p["step"]), w.attn_mult, w.softcap)
    out = U.host(st())
    torch.cuda.synchronize()
    assert st.status.item() == 0
    B, T, Hq, Hkv, D = w.B, w.T, w.Hq, w.Hkv, w.D
    to64 = orc.bf16_bits_to_f64
    g = gi.rng(4343)
    errs = []
    for b in range(B):
        o = int(p["step"][b])
        pos = (o + np.arange(T))[None]
        qr = orc.rope(to64(p["q"][b:b + 1]), pos, out="bf16")
        kr = orc.rope(to64(p["k_new"][b:b + 1]), pos, out="bf16")
        k64 = np.concatenate([to64(p["k_cache"][b:b + 1, :o]), kr], axis=1)
        v64 = np.concatenate([to64(p["v_cache"][b:b + 1, :o]), to64(p["v_new"][b:b + 1])], axis=1)
        for t in [0, T - 1] + list(g.integers(0, T, 2)):
            mask_row = np.arange(o + T) <= o + t
            ref = np.concatenate([orc.attention_rows(qr, k64, v64, 0, t, h, mask_row, w.attn_mult, w.softcap)
                                  for h in range(Hq)])
            errs.append(U.assert_bf16_close(out[b, t], ref, f"chunk b={b} (offset {o}) t={t}"))
    print(f"chunk sampled rows, max abs err {max(errs):.2e}")


def test_moe_b4_t2048_sampled(G):
    """The MoE FFN sub-layer at its full size (8192 token rows, d 6144, F 32768,
    8 experts, top-2): the routing of every row is a valid top-2 of the oracle's
    probabilities with the oracle's gates, and sampled rows match the oracle
    run on those rows with the same expert choice."""
    grok, pipe, U, torch = G
    w = gi.WORKLOADS["moe_b4_t2048"]
    p = gi.make_workload(w.name)
    T, d = w.B * w.T, w.d_model
    xb = p["x"].reshape(T, d)
    x = U.dev_bf16(xb)
    experts = [tuple(U.dev(a) for a in ex) for ex in p["experts"]]
    step = pipe.MoeStep(x, U.dev(p["w_router"]), experts, k=w.top_k)
    del experts
    y = U.host(step())
    torch.cuda.synchronize()
    print("moe: GPU step done", flush=True)
    idx = step.idx.cpu().numpy().astype(np.int64)
    gates = step.gates.cpu().numpy()
    x64 = orc.bf16_bits_to_f64(xb)
    n = orc.rmsnorm(x64, None, w.eps, out="bf16")
    probs, _, _ = orc.moe_route(n, p["w_router"], w.top_k)
    kth = -np.sort(-probs, axis=1)[:, w.top_k - 1]
    chosen = np.take_along_axis(probs, idx, axis=1)
    assert np.all((idx >= 0) & (idx < w.n_experts)) and np.all(idx[:, 0] != idx[:, 1])
    # the GPU routes its own normalised rows, which may differ from the oracle's
    # by one bf16 rounding in a few elements: probabilities agree to ~1e-4
    assert np.all(chosen >= kth[:, None] - 1e-3)
    gerr = np.abs(gates - chosen).max()
    assert gerr <= 1e-3, gerr
    print(f"moe: max gate error {gerr:.2e}", flush=True)
    counts = np.bincount(idx.ravel(), minlength=w.n_experts)
    print(f"moe: routing valid, rows per expert {counts.tolist()}", flush=True)
    rows = np.array([0, T - 1] + list(gi.rng(4444).integers(1, T - 1, 2)))
    ref, _, _ = orc.moe_sublayer(x64[rows], p["w_router"], p["experts"], w.eps, w.top_k, idx=idx[rows])
    # y = x + n(mix): the relative part of the bound belongs to the larger of
    # |y| and the normalised summand, here ref - x (exact up to ref's rounding)
    nm = ref - x64[rows]
    err = U.assert_bf16_close(y[rows], ref, "moe sampled rows", magnitude=np.maximum(np.abs(ref), np.abs(nm)))
    print(f"moe sampled rows {rows.tolist()}: max abs err {err:.2e}, rel L2 {U.rel_l2(y[rows], ref):.2e}")
