"""Replaying a HIP graph of a hot-path step gives the same bits as running the
step eagerly, on every replay, with eager work in between (the benchmark times
graph replays)."""
import math

import numpy as np
import pytest

import gqa_inputs as gi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gqa_attention_grok_amd.pipeline as pipe
    import gpu_util
    return pipe, gpu_util, torch


def test_decode_step_graph_replays_match_eager(G):
    pipe, U, torch = G
    B, Hq, Hkv, D, Tmax = 3, 48, 8, 128, 2048
    d = gi.make_decode_inputs(B, Hq, Hkv, D, Tmax, seed=21, lengths=[1, 700, 2048])
    kc, vc = U.dev_bf16(d["k_cache"]), U.dev_bf16(d["v_cache"])
    q0 = U.dev_bf16(d["q"])
    q = q0.clone()
    st = pipe.DecodeStep(kc, vc, q, U.dev_bf16(d["k_new"]), U.dev_bf16(d["v_new"]), U.dev(d["step"]),
                         1 / math.sqrt(D))
    eager = U.bits(st())
    graph = pipe.capture(st)
    for rep in range(3):
        q.copy_(q0)              # the step rotates q in place: restore its input
        st.out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(U.bits(st.out), eager, err_msg=f"replay {rep}")


def test_prefill_step_graph_replays_match_eager(G):
    pipe, U, torch = G
    p = gi.make_prefill_inputs(1, 200, 48, 8, 128, seed=22)
    q0, k0 = U.dev_bf16(p["q"]), U.dev_bf16(p["k"])
    q, k = q0.clone(), k0.clone()
    st = pipe.PrefillStep(q, k, U.dev_bf16(p["v"]), 4 / math.sqrt(128))
    eager = U.bits(st())
    fused = pipe.PrefillStep(q0.clone(), k0.clone(), U.dev_bf16(p["v"]), 4 / math.sqrt(128), fused_rope=True)
    np.testing.assert_array_equal(U.bits(fused()), eager)  # q rotated in the kernel: the same bits
    graph = pipe.capture(st)
    for rep in range(3):
        q.copy_(q0)
        k.copy_(k0)
        st.out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(U.bits(st.out), eager, err_msg=f"replay {rep}")
