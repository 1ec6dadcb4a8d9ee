"""The autograd wrapper on the GPU: forward and gradients against the oracle,
for the batch and the packed forms."""
import numpy as np
import pytest

import context_attention_flash_amd as ca
import oracle
from context_attention_flash_amd import synth
from context_attention_flash_amd.autograd import ring_flash_attn_func, ring_flash_attn_varlen_func

from _helpers import max_err_lse, say, shard, to_dev, tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _leaf(x, dtype):
    return to_dev(x, dtype).requires_grad_(True)


def _check(w, glob, rank, out, lse, dq, dk, dv):
    sh = shard(glob, w, rank)
    ref_out, ref_lse = oracle.rank_share_forward(glob["q"], glob["k"], glob["v"], w.layout,
                                                 w.world, rank, w.causal, w.cu_seqlens,
                                                 window=w.window)
    t = tol(w.dtype)
    assert float(np.abs(out - ref_out).max()) <= t["out"]
    assert max_err_lse(lse, ref_lse) <= t["lse"]
    rdq, rdk, rdv = oracle.rank_share_backward(glob["q"], glob["k"], glob["v"], sh["dout"],
                                               w.layout, w.world, rank, w.causal, w.cu_seqlens,
                                               window=w.window)
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e, bound = float(np.abs(got - ref).max()), 5e-2 * float(np.abs(ref).max())
        assert e <= bound, (name, e, bound)


@pytest.mark.parametrize("layout,causal,window", [
    (ca.BASIC, True, (-1, -1)), (ca.ZIGZAG, True, (120, -1)), (ca.STRIPE, False, (-1, -1))])
def test_batch_form(layout, causal, window):
    w = synth.Workload("ag-batch", 2, 4, 2, 128, 4 * 160, 4, 0, causal, layout, "bf16",
                       seed=90 + layout, with_grad=True, window=window)
    glob = synth.draw_global(w)
    for rank in (0, 3):
        say(f"autograd batch layout={layout} causal={causal} window={window} rank={rank}")
        sh = shard(glob, w, rank)
        q, k, v = (_leaf(sh[n], "bf16") for n in ("q", "k", "v"))
        out, lse, _ = ring_flash_attn_func(q, k, v, causal=causal, window_size=window,
                                           return_attn_probs=True, world=4, rank=rank,
                                           layout=layout)
        out.backward(to_dev(sh["dout"], "bf16"))
        torch.cuda.synchronize()
        assert q.grad.dtype == torch.bfloat16 and k.grad.shape == k.shape
        _check(w, glob, rank, out.detach().float().cpu().numpy(), lse.cpu().numpy(),
               q.grad.float().cpu().numpy(), k.grad.float().cpu().numpy(),
               v.grad.float().cpu().numpy())


@pytest.mark.parametrize("layout,window", [
    (ca.VARLEN_RING, (-1, -1)), (ca.VARLEN_ZIGZAG, (90, -1)), (ca.LLAMA3, (-1, -1))])
def test_varlen_form(layout, window):
    D, S = 4, 192
    N = D * S
    cu = synth.random_cu_seqlens(N, 3, np.random.default_rng(5 + layout),
                                 multiple=synth.doc_multiple(layout, D))
    w = synth.Workload("ag-varlen", 1, 4, 2, 64, N, D, 0, True, layout, "bf16", seed=95 + layout,
                       cu_seqlens=tuple(cu), with_grad=True, window=window)
    glob = synth.draw_global(w)
    for rank in (1, 3):
        say(f"autograd varlen layout={layout} window={window} rank={rank}")
        sh = shard(glob, w, rank)
        q, k, v = (_leaf(sh[n][..., 0, :, :, :] if n != "q" else sh[n][0], "bf16")
                   for n in ("q", "k", "v"))
        out, lse, _ = ring_flash_attn_varlen_func(q, k, v, cu, max_seqlen=None, causal=True,
                                                  window_size=window, return_attn_probs=True,
                                                  world=D, rank=rank, layout=layout)
        assert out.shape == q.shape
        out.backward(to_dev(sh["dout"][0], "bf16"))
        torch.cuda.synchronize()
        _check(w, glob, rank, out.detach().float().cpu().numpy()[None], lse.cpu().numpy()[None],
               q.grad.float().cpu().numpy()[None], k.grad.float().cpu().numpy()[:, None],
               v.grad.float().cpu().numpy()[:, None])


def test_wrapper_output_equals_c_abi_call():
    w = synth.Workload("ag-same", 1, 4, 4, 128, 4 * 128, 4, 2, True, ca.BASIC, "bf16", seed=99)
    glob = synth.draw_global(w)
    sh = shard(glob, w, 2)
    q, k, v = (to_dev(sh[n], "bf16") for n in ("q", "k", "v"))
    say("autograd wrapper vs direct call")
    a = ring_flash_attn_func(q, k, v, causal=True, world=4, rank=2)
    b, _ = ca.ring_attn_fwd(ca.desc_from_workload(w), q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
