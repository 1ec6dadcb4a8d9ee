"""The no-allocation backward entry point (ring_attn_bwd_noalloc) against the
ordinary one (ring_attn_bwd), through the C ABI, on two calls in a row (the
second smaller), each also against the fp64 oracle; plus its refusals."""
import ctypes

import numpy as np
import pytest

import context_attention_flash_amd as ca
import oracle
from context_attention_flash_amd import synth

from _helpers import say, shard, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _case(layout, D, S, Hq, Hkv, d, causal, seed, rank):
    N = D * S
    cu = None
    if layout in synth.VARLEN_LAYOUTS:
        cu = tuple(synth.random_cu_seqlens(N, 3, np.random.default_rng(seed),
                                           multiple=synth.doc_multiple(layout, D)))
    w = synth.Workload(f"noalloc-{layout}", 1, Hq, Hkv, d, N, D, rank, causal, layout, "bf16",
                       seed=seed, cu_seqlens=cu, with_grad=True)
    glob = synth.draw_global(w)
    sh = shard(glob, w, rank)
    desc = ca.desc_from_workload(w)
    dev = {n: to_dev(sh[n], "bf16") for n in ("q", "k", "v", "dout")}
    return w, glob, sh, desc, dev


def _check_against_oracle(w, glob, sh, dq, dk, dv):
    rdq, rdk, rdv = oracle.rank_share_backward(glob["q"], glob["k"], glob["v"], sh["dout"], w.layout,
                                               w.world, w.rank, w.causal, w.cu_seqlens)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e = float(np.abs(got.cpu().numpy() - ref).max())
        assert e <= 5e-2 * float(np.abs(ref).max()), (name, e)


def test_noalloc_matches_ordinary_backward_twice():
    assert ca.ring_attn_noalloc_scratch_bytes() == 64 << 20
    cases = [(ca.ZIGZAG, 4, 640, 4, 2, 128, True, 11, 1),     # first call
             (ca.BASIC, 4, 200, 2, 2, 64, True, 12, 3)]       # second, smaller
    for layout, D, S, Hq, Hkv, d, causal, seed, rank in cases:
        say(f"noalloc layout={layout} S={S} Hq={Hq} d={d} rank={rank}")
        w, glob, sh, desc, dev = _case(layout, D, S, Hq, Hkv, d, causal, seed, rank)
        # an ordinary call builds and caches the plan of the shape
        out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"], w.cu_seqlens)
        ref = ca.ring_attn_bwd(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse,
                               w.cu_seqlens)
        dq = torch.full_like(ref[0], float("nan"))
        dk = torch.zeros_like(ref[1])
        dv = torch.zeros_like(ref[2])
        ca.ring_attn_bwd_noalloc(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse,
                                 dq, dk, dv, w.cu_seqlens)
        torch.cuda.synchronize()
        for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            e = float((got - want).abs().max())
            assert e <= 5e-2 * float(want.abs().max()), (name, e)
        _check_against_oracle(w, glob, sh, dq, dk, dv)


def test_noalloc_refusals():
    fake = ctypes.c_void_p(0x1000)
    # a descriptor whose minimum workspace exceeds the static array
    big = ca.make_desc(1, 32, 32, 128, 8 * 8192, 8, 7, True, ca.BASIC)
    rc = ca.lib().ring_attn_bwd_noalloc(ctypes.byref(big), *([fake] * 6), None, fake, fake, fake,
                                        None)
    assert rc == -13 and "scratch" in ca.ring_attn_strerror(rc)
    # a shape with no cached plan: refused before any device work
    w, glob, sh, desc, dev = _case(ca.STRIPE, 4, 136, 2, 1, 64, True, 13, 2)
    out = torch.zeros_like(dev["q"])
    lse = torch.zeros(1, 2, 136, device="cuda")
    dq = torch.zeros(dev["q"].shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(dev["k"].shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(dev["v"].shape, dtype=torch.float32, device="cuda")
    ca.ring_attn_clear_cache()
    with pytest.raises(ca.RingAttnError, match="RA_E_NO_PLAN"):
        ca.ring_attn_bwd_noalloc(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse,
                                 dq, dk, dv)
