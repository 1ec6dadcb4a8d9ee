"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (fused merge), on outputs the oracle can afford to compute: sampled query
rows x heads for the forward and dq, and the complete dK/dV of one KV head for
the backward (the oracle sums that head's contributions over every query row of
the rank, chunk by chunk)."""
import numpy as np
import pytest

import context_attention_flash_amd as ca
import oracle
from context_attention_flash_amd import synth

from _helpers import max_err_lse, say, to_dev, tol

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _inputs(w):
    g = synth.draw_global(w)
    desc = ca.desc_from_workload(w)
    cu = list(w.cu_seqlens) if w.cu_seqlens else None
    pos_q = oracle.positions(w.layout, w.seqlen, w.world, w.rank, cu)
    nb = oracle.num_blocks(w.layout, w.world)
    blocks = [oracle.kv_positions(w.layout, w.seqlen, w.world, j, cu) for j in range(nb)]
    dev = {"q": to_dev(g["q"][:, pos_q], w.dtype),
           "k": to_dev(np.stack([g["k"][:, p] for p in blocks]), w.dtype),
           "v": to_dev(np.stack([g["v"][:, p] for p in blocks]), w.dtype)}
    if w.with_grad:
        dev["dout"] = to_dev(g["dout"][:, pos_q], w.dtype)
    return g, desc, cu, pos_q, dev


def _sample_rows(S, rng, extra=()):
    rows = {0, 1, 63, 64, 127, 128, S // 2, S // 2 - 1, S - 1, S - 2, S - 128, *extra}
    rows |= set(int(x) for x in rng.integers(0, S, 24))
    return np.array(sorted(r for r in rows if 0 <= r < S))


@pytest.mark.parametrize("name", ["basic_s4096", "zigzag", "llama3", "basic_s8192"])
def test_workload_forward(name):
    w = synth.WORKLOADS[name]
    say(f"workload fwd {name}")
    g, desc, cu, pos_q, dev = _inputs(w)
    out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"], w.cu_seqlens)
    torch.cuda.synchronize()
    S = w.shard
    extra = ()
    if w.layout == ca.ZIGZAG:
        extra = (S // 2 - 1, S // 2, S // 2 + 1)
    if cu is not None:  # rows at document boundaries inside the shard
        extra = tuple(int(c - pos_q[0]) + o for c in cu for o in (-1, 0, 1))
    rows = _sample_rows(S, np.random.default_rng(5), extra)
    heads = sorted({0, w.heads_q // 2 + 1, w.heads_q - 1})
    ref_out, ref_lse = oracle.rank_share_forward(g["q"], g["k"], g["v"], w.layout, w.world, w.rank,
                                                 w.causal, cu, rows=rows, heads=heads)
    got_out = out[:, torch.tensor(rows)].float().cpu().numpy()
    got_lse = lse[:, :, torch.tensor(rows)].cpu().numpy()
    t = tol(w.dtype)
    for h in heads:
        e_out = float(np.abs(got_out[:, :, h] - ref_out[:, :, h]).max())
        e_lse = max_err_lse(got_lse[:, h], ref_lse[:, h])
        assert e_out <= t["out"], (h, e_out)
        assert e_lse <= t["lse"], (h, e_lse)
    assert torch.isfinite(out.float()).all().item()
    assert torch.isfinite(lse).all().item()


def test_workload_backward_basic_s8192():
    w = synth.WORKLOADS["basic_s8192"]
    say("workload bwd basic_s8192")
    g, desc, cu, pos_q, dev = _inputs(w)
    out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"])
    dq, dk, dv = ca.ring_attn_bwd(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse)
    torch.cuda.synchronize()
    dout_local = g["dout"][:, pos_q]
    S = w.shard
    # dq on sampled rows x heads (each row's dq depends on that row only)
    rows = _sample_rows(S, np.random.default_rng(6))
    heads = [0, 17, 31]
    rdq, _, _ = oracle.rank_share_backward(g["q"], g["k"], g["v"], dout_local, w.layout, w.world,
                                           w.rank, w.causal, rows=rows, heads=heads)
    got_dq = dq[:, torch.tensor(rows)].cpu().numpy()
    for h in heads:
        ref = rdq[:, :, h]
        assert np.abs(got_dq[:, :, h] - ref).max() <= 5e-2 * np.abs(ref).max()
    # the complete dK/dV of KV head 5, summed over every query row of the rank
    hk = 5
    rdk = rdv = None
    for a in range(0, S, 1024):
        _, ck, cv = oracle.rank_share_backward(g["q"], g["k"], g["v"], dout_local, w.layout,
                                               w.world, w.rank, w.causal,
                                               rows=np.arange(a, min(S, a + 1024)), heads=[hk])
        rdk = ck[..., hk, :] if rdk is None else rdk + ck[..., hk, :]
        rdv = cv[..., hk, :] if rdv is None else rdv + cv[..., hk, :]
    got_dk = dk[..., hk, :].cpu().numpy()
    got_dv = dv[..., hk, :].cpu().numpy()
    assert np.abs(got_dk - rdk).max() <= 5e-2 * np.abs(rdk).max()
    assert np.abs(got_dv - rdv).max() <= 5e-2 * np.abs(rdv).max()
    # blocks this rank never sees stay untouched (causal basic: none here, rank 7)
    assert torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()


@pytest.mark.parametrize("name", ["zigzag", "llama3"])
def test_workload_backward_dq_sampled(name):
    """The backward at the zigzag (GQA 32/8, 16384-row shard) and llama3
    (packed, one step over the gathered 65536 keys) sizes, through the stored-dS
    path the bench uses: dq on sampled rows x heads (each row's dq depends on
    that row alone); dk, dv finite."""
    w = synth.WORKLOADS[name].replace(with_grad=True)
    say(f"workload bwd {name}")
    g, desc, cu, pos_q, dev = _inputs(w)
    ws = ca.alloc_workspace(desc, True, cu_seqlens=cu)
    assert ws.numel() >= ca.ring_attn_workspace_bytes(desc, True) + ca.ring_attn_bwd_ds_bytes(desc, cu)
    out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"], cu)
    dq, dk, dv = ca.ring_attn_bwd(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, cu,
                                  workspace=ws)
    torch.cuda.synchronize()
    rows = _sample_rows(w.shard, np.random.default_rng(8))
    heads = [0, 13, 31]
    rdq, _, _ = oracle.rank_share_backward(g["q"], g["k"], g["v"], g["dout"][:, pos_q], w.layout,
                                           w.world, w.rank, w.causal, cu, rows=rows, heads=heads)
    got = dq[:, torch.tensor(rows)].cpu().numpy()
    for h in heads:
        ref = rdq[:, :, h]
        assert np.abs(got[:, :, h] - ref).max() <= 5e-2 * np.abs(ref).max(), h
    assert torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()
