"""The allocation-free decode step (grok_attn_decode_append_noalloc, split
partials in the library's per-GPU scratch array) against the workspace form
(grok_attn_decode_append) on the same inputs: identical outputs, rotated q,
new_step and cache writes, bit for bit, on two calls in a row -- the ragged
32-sequence decode at full size, then a smaller ragged batch, so the second
call runs over the first one's leftover scratch contents."""
import math

import numpy as np
import pytest

import gqa_inputs as gi

pytestmark = pytest.mark.gpu


def _compare(grok, torch, dev_bf16, dev, p, attn_mult, softcap=30.0):
    B, _, Hq, D = p["q"].shape
    Tmax, Hkv = p["k_cache"].shape[1], p["k_cache"].shape[2]
    q, kn, vn, step = dev_bf16(p["q"]), dev_bf16(p["k_new"]), dev_bf16(p["v_new"]), dev(p["step"])
    res = []
    for noalloc in (False, True):
        kc, vc = dev_bf16(p["k_cache"]), dev_bf16(p["v_cache"])
        out = torch.empty((B, 1, Hq * D), dtype=torch.bfloat16, device="cuda")
        q_out = torch.empty_like(q)
        new_step = torch.empty(B, dtype=torch.int32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if noalloc:
            grok.grok_attn_decode_append_noalloc(q, kn, vn, kc, vc, step, out, attn_mult, softcap,
                                                 new_step=new_step, q_out=q_out, status=status)
        else:
            ws = torch.zeros(grok.grok_attn_decode_workspace_bytes(B, Tmax, Hq, Hkv, D), dtype=torch.uint8,
                             device="cuda")
            grok.grok_attn_decode_append(q, kn, vn, kc, vc, step, out, ws, attn_mult, softcap,
                                         new_step=new_step, q_out=q_out, status=status)
        torch.cuda.synchronize()
        res.append((out, q_out, new_step, status, kc, vc))
    (o1, qo1, ns1, st1, kc1, vc1), (o2, qo2, ns2, st2, kc2, vc2) = res
    assert st1.item() == 0 and st2.item() == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "attention output differs"
    assert torch.equal(qo1.view(torch.int16), qo2.view(torch.int16)), "rotated q differs"
    assert torch.equal(ns1, ns2) and np.array_equal(ns2.cpu().numpy(), p["step"] + 1)
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "k cache differs"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "v cache differs"
    # not a trivial output: the rows are finite and not all zero
    o = o2.float()
    assert torch.isfinite(o).all() and o.abs().amax().item() > 0


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch
    assert torch.cuda.is_available()
    import gqa_attention_grok_amd as grok
    from gqa_inputs.device import dev, dev_bf16
    w = gi.WORKLOADS["decode_ragged_b32_t8192"]
    p = gi.make_workload(w.name)
    need = grok.grok_attn_decode_workspace_bytes(w.B, w.Tmax, w.Hq, w.Hkv, w.D)
    assert need <= grok.grok_attn_decode_append_noalloc_max_bytes()
    print(f"noalloc call 1: ragged decode B={w.B} Tmax={w.Tmax} ({need} scratch bytes)", flush=True)
    _compare(grok, torch, dev_bf16, dev, p, w.attn_mult, w.softcap)
    del p
    # a smaller call right after: fewer sequences, shorter cache, other lengths
    p = gi.make_decode_inputs(3, 48, 8, 128, 1024, seed=777, lengths=[1, 300, 1024])
    print("noalloc call 2: B=3 Tmax=1024 lengths 1, 300, 1024", flush=True)
    _compare(grok, torch, dev_bf16, dev, p, 1.0 / math.sqrt(128))
