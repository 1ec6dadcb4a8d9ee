"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (fused merge), on outputs the oracle can afford to compute: sampled query
rows x heads for the forward and dq; the complete dK/dV of one KV head for the
backward (the oracle sums that head's contributions over every query row of
the rank, chunk by chunk); and the complete dK/dV of every KV head when dout
is zero outside sampled rows."""
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
    heads = list(range(w.heads_q))   # every q head (and so every kv head) on the sampled rows
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
    heads = list(range(w.heads_q))
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
    assert torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()
    _check_dv_sums(w, dout_local, dk, dv)


def _check_dv_sums(w, dout_local, dk, dv):
    """Properties of the complete dK/dV that hold at any size, per kv head:
    the softmax rows sum to one, so the dV rows of a kv head, summed over
    every block and key, equal the dout rows of its q heads summed over the
    rank's rows; and dS = P (dP - Delta) sums to zero over the keys of a row,
    so the dK rows of a kv head sum to zero.  A kv-head (GQA group) indexing
    error in the dK/dV kernels or in the dS store breaks the first."""
    group = w.heads_q // w.heads_kv
    dv64 = dv.double().sum(dim=(0, 2)).cpu().numpy()          # [B, Hkv, d]
    dk_sum = dk.double().sum(dim=(0, 2)).cpu().numpy()
    dk_abs = dk.double().abs().sum(dim=(0, 2)).cpu().numpy()
    do = dout_local.astype(np.float64).reshape(w.batch, -1, w.heads_kv, group, w.head_dim)
    ref = do.sum(axis=(1, 3))                                 # [B, Hkv, d]
    assert np.abs(dv64 - ref).max() <= 2e-2 * np.abs(ref).max(), np.abs(dv64 - ref).max()
    assert np.all(np.abs(dk_sum) <= 1e-2 * dk_abs + 1e-3)


@pytest.mark.parametrize("name", ["zigzag", "llama3"])
def test_workload_backward_full_size(name):
    """The backward at the zigzag (GQA 32/8, 16384-row shard) and llama3
    (packed, one step over the gathered 65536 keys) sizes, through the stored-dS
    path the bench uses: dq of every q head on sampled rows (each row's dq
    depends on that row alone); the dV/dK sums over keys of every kv head; and
    for llama3 the complete dK/dV of one kv head (its 4 q heads, every query row
    of the rank), with the oracle's sums restricted to the keys the rank's
    documents hold."""
    w = synth.WORKLOADS[name].replace(with_grad=True)
    say(f"workload bwd {name}")
    g, desc, cu, pos_q, dev = _inputs(w)
    ws = ca.alloc_workspace(desc, True, cu_seqlens=cu)
    assert ws.numel() >= ca.ring_attn_workspace_bytes(desc, True) + ca.ring_attn_bwd_ds_bytes(desc, cu)
    out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"], cu)
    dq, dk, dv = ca.ring_attn_bwd(desc, dev["dout"], dev["q"], dev["k"], dev["v"], out, lse, cu,
                                  workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()
    dout_local = g["dout"][:, pos_q]
    rows = _sample_rows(w.shard, np.random.default_rng(8))
    heads = list(range(w.heads_q))
    rdq, _, _ = oracle.rank_share_backward(g["q"], g["k"], g["v"], dout_local, w.layout,
                                           w.world, w.rank, w.causal, cu, rows=rows, heads=heads)
    got = dq[:, torch.tensor(rows)].cpu().numpy()
    for h in heads:
        ref = rdq[:, :, h]
        assert np.abs(got[:, :, h] - ref).max() <= 5e-2 * np.abs(ref).max(), h
    _check_dv_sums(w, dout_local, dk, dv)
    if w.layout == ca.LLAMA3:
        # keys the rank's rows can see: from the start of the first document
        # that overlaps the shard to the shard's end
        k0 = max(c for c in cu if c <= pos_q[0])
        k1 = int(pos_q[-1]) + 1
        hk = 5
        group = w.heads_q // w.heads_kv
        rdk = rdv = None
        for a in range(0, w.shard, 2048):
            _, ck, cv = oracle.rank_share_backward(
                g["q"], g["k"], g["v"], dout_local, w.layout, w.world, w.rank, w.causal, cu,
                rows=np.arange(a, min(w.shard, a + 2048)),
                heads=list(range(hk * group, (hk + 1) * group)), key_range=(k0, k1))
            rdk = ck[..., hk, :] if rdk is None else rdk + ck[..., hk, :]
            rdv = cv[..., hk, :] if rdv is None else rdv + cv[..., hk, :]
        got_dk = dk[..., hk, :].cpu().numpy()
        got_dv = dv[..., hk, :].cpu().numpy()
        assert np.abs(got_dk - rdk).max() <= 5e-2 * np.abs(rdk).max()
        assert np.abs(got_dv - rdv).max() <= 5e-2 * np.abs(rdv).max()


@pytest.mark.parametrize("name", ["zigzag", "llama3", "basic_s8192"])
def test_workload_backward_dkdv_from_sampled_rows(name):
    """The complete dK/dV of every kv head at the zigzag, llama3 and
    basic_s8192 sizes.
    dK and dV are linear in dout, and a row whose dout is zero adds nothing to
    them (its dP and Delta are zero, so its dS = P (dP - Delta) is too): with
    dout zero except on sampled rows, every element of the GPU's dK/dV (all
    blocks, keys and kv heads, every q head of each group) must equal the
    oracle's sums over those rows alone."""
    w = synth.WORKLOADS[name].replace(with_grad=True)
    say(f"workload bwd dk/dv from sampled rows {name}")
    g, desc, cu, pos_q, dev = _inputs(w)
    S = w.shard
    extra = (S // 2 - 1, S // 2, S // 2 + 1) if w.layout == ca.ZIGZAG else ()
    if cu is not None:
        extra = tuple(int(c - pos_q[0]) + o for c in cu for o in (-1, 0, 1))
    rows = _sample_rows(S, np.random.default_rng(11), extra)
    dout_local = np.zeros_like(g["dout"][:, pos_q])
    dout_local[:, rows] = g["dout"][:, pos_q][:, rows]
    dout = to_dev(dout_local, w.dtype)
    ws = ca.alloc_workspace(desc, True, cu_seqlens=cu)
    out, lse = ca.ring_attn_fwd(desc, dev["q"], dev["k"], dev["v"], cu)
    _, dk, dv = ca.ring_attn_bwd(desc, dout, dev["q"], dev["k"], dev["v"], out, lse, cu, workspace=ws)
    torch.cuda.synchronize()
    # (the drawn inputs hold bf16 values exactly: both sides see the same dout)
    _, rdk, rdv = oracle.rank_share_backward(g["q"], g["k"], g["v"], dout_local, w.layout, w.world,
                                             w.rank, w.causal, cu, rows=rows,
                                             heads=list(range(w.heads_q)))
    got_dk, got_dv = dk.cpu().numpy(), dv.cpu().numpy()
    assert got_dk.shape == rdk.shape and got_dv.shape == rdv.shape
    assert np.abs(got_dk - rdk).max() <= 5e-2 * np.abs(rdk).max(), np.abs(got_dk - rdk).max()
    assert np.abs(got_dv - rdv).max() <= 5e-2 * np.abs(rdv).max(), np.abs(got_dv - rdv).max()
    # the rows' contributions reach keys of every kv head
    assert np.abs(rdv).reshape(-1, w.heads_kv, w.head_dim).max(axis=(0, 2)).min() > 0
