"""GPU parity of the attention forward with an int8 P.V product
(brq_attn_fwd) against the oracle, bit for bit: head dims 64 and 128,
grouped-query head maps, plain causal and sliding windows (1, 64, a window
that is not a block multiple), the flushing path for tiny logits inputs,
and the Open-1B attention shape (16 query heads over 4 key/value heads,
4096 tokens, head dim 128, window 512 and fully causal) on sampled heads.
"""
import sys

import numpy as np
import pytest
import torch

import brq_synth as syn
import oracle as orc
from tests.gpu_util import DEV, assert_bitwise, to_dev

pytestmark = pytest.mark.gpu

brq = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global brq
    import bitwise_reproducible_int8_amd as m
    m.lib()
    brq = m
    yield


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def qkv(Hq, Hkv, T, d, tag, q_std=1.0):
    q = syn.normal((Hq, T, d), q_std, tag=tag, bf16=True)
    k = syn.normal((Hkv, T, d), 1.0, tag=tag + 1, bf16=True)
    v = syn.normal((Hkv, T, d), 1.0, tag=tag + 2, bf16=True)
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv,T,d,window", [(4, 1, 128, 64, None), (4, 4, 64, 128, None),
                                               (4, 2, 256, 128, 64), (2, 1, 192, 64, 1),
                                               (8, 2, 320, 128, 100), (4, 1, 256, 64, 1000)])
def test_attn_fwd(Hq, Hkv, T, d, window):
    say("attn_fwd", Hq, Hkv, T, d, window)
    q, k, v = qkv(Hq, Hkv, T, d, 341)
    o, fl = orc.attn_fwd(q, k, v, window)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    go = brq.attn_fwd(to_dev(q), to_dev(k), to_dev(v), window, flags=flags)
    assert_bitwise(go, o, "o")
    assert int(flags.item()) == fl == 0


def test_attn_fwd_flushing_form():
    """Query values near 2^-122: products and partial sums can be subnormal,
    so the logits take the flushing form (and the softmax of such tiny
    logits is nearly uniform)."""
    say("attn_fwd_flushing_form")
    q, k, v = qkv(2, 1, 128, 64, 344, q_std=3e-37)
    o, _ = orc.attn_fwd(q, k, v, None)
    go = brq.attn_fwd(to_dev(q), to_dev(k), to_dev(v))
    assert_bitwise(go, o, "o tiny q")


def test_attn_fwd_repeat_and_edges():
    say("attn_fwd_repeat_and_edges")
    q, k, v = qkv(4, 2, 128, 128, 347)
    a = brq.attn_fwd(to_dev(q), to_dev(k), to_dev(v), 64)
    b = brq.attn_fwd(to_dev(q), to_dev(k), to_dev(v), 64)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    with pytest.raises(brq.BrqError):  # T not a multiple of 64
        brq.attn_fwd(to_dev(q[:, :100]), to_dev(k[:, :100]), to_dev(v[:, :100]))
    with pytest.raises(brq.BrqError):  # head dim outside {64, 128}
        brq.attn_fwd(to_dev(q[:, :, :32]), to_dev(k[:, :, :32]), to_dev(v[:, :, :32]))
    e = torch.empty((4, 0, 128), dtype=torch.bfloat16, device=DEV)
    assert brq.attn_fwd(e, e[:2], e[:2]).shape == (4, 0, 128)


@pytest.mark.parametrize("window", [512, None])
def test_attn_fwd_open1b_shape(window):
    """16 query heads over 4 key/value heads, 4096 tokens, head dim 128: the
    GPU runs every head; the oracle recomputes query heads 0 and 13 (their
    key/value heads 0 and 3) in full."""
    say("attn_fwd_open1b", window)
    Hq, Hkv, T, d = 16, 4, 4096, 128
    q, k, v = qkv(Hq, Hkv, T, d, 350)
    go = brq.attn_fwd(to_dev(q), to_dev(k), to_dev(v), window).cpu().numpy()
    for h in (0, 13):
        g = h // (Hq // Hkv)
        o, fl = orc.attn_fwd(q[h:h + 1], k[g:g + 1], v[g:g + 1], window)
        assert_bitwise(go[h], o[0], f"o head {h}")
        assert fl == 0
