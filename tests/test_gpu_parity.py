"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded inputs that span several tiles and a ragged tail.

Tolerances: fp32 out/lse <= 1e-4; bf16 out <= 2e-2, lse <= 1e-3; gradients
max-abs-err <= 5e-2 * max |oracle grad| per tensor.
"""
import numpy as np
import pytest

import context_attention_flash_amd as ca
import oracle
from context_attention_flash_amd import synth

from _helpers import max_err_lse, say, shard, to_dev, tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
LAYOUTS = [ca.BASIC, ca.ZIGZAG, ca.STRIPE, ca.VARLEN_RING, ca.LLAMA3, ca.VARLEN_ZIGZAG,
           ca.VARLEN_STRIPE]


def _small_workload(layout, causal, head_dim, dtype="bf16", D=4, S=200, B=2, Hq=4, Hkv=2,
                    seed=0, with_grad=False, window=(-1, -1)):
    N = D * S
    cu = None
    if layout in (ca.VARLEN_RING, ca.VARLEN_ZIGZAG, ca.VARLEN_STRIPE):
        cu = tuple(synth.random_cu_seqlens(N, 3, np.random.default_rng(seed + 7),
                                           multiple=synth.doc_multiple(layout, D)))
        B = 1
    elif layout == ca.LLAMA3:
        cu = tuple(synth.random_cu_seqlens(N, 4, np.random.default_rng(seed + 7)))
        B = 1
    return synth.Workload(f"small-{layout}", B, Hq, Hkv, head_dim, N, D, 0, causal, layout, dtype,
                          seed=seed, cu_seqlens=cu, with_grad=with_grad, window=window)


def _run_fwd(w, glob, rank, merge_mode=ca.RA_MERGE_FUSED):
    sh = shard(glob, w, rank)
    desc = ca.desc_from_workload(w, rank=rank, merge_mode=merge_mode)
    q, k, v = (to_dev(sh[n], w.dtype) for n in ("q", "k", "v"))
    out, lse = ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens)
    torch.cuda.synchronize()
    return sh, desc, (q, k, v), out.float().cpu().numpy(), lse.cpu().numpy()


def _check_fwd(w, glob, rank, out, lse, ref=None):
    """out and lse against the oracle's rank share (`ref`: the oracle's
    (out, lse) when the caller has it already)."""
    ref_out, ref_lse = ref if ref is not None else oracle.rank_share_forward(
        glob["q"], glob["k"], glob["v"], w.layout, w.world, rank, w.causal, w.cu_seqlens,
        window=w.window)
    t = tol(w.dtype)
    e_out = float(np.abs(out - ref_out).max())
    e_lse = max_err_lse(lse, ref_lse)
    assert e_out <= t["out"], e_out
    assert e_lse <= t["lse"], e_lse
    return e_out, e_lse


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("merge_mode", [ca.RA_MERGE_FUSED, ca.RA_MERGE_SEPARATE,
                                        ca.RA_MERGE_STEPWISE])
def test_fwd_bf16_small(layout, causal, head_dim, merge_mode):
    w = _small_workload(layout, causal, head_dim, seed=layout * 4 + causal)
    glob = synth.draw_global(w)
    for rank in (0, 2, w.world - 1):
        say(f"fwd bf16 layout={layout} causal={causal} d={head_dim} merge={merge_mode} rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank, merge_mode)
        _check_fwd(w, glob, rank, out, lse)


@pytest.mark.parametrize("layout", [ca.BASIC, ca.STRIPE, ca.LLAMA3])
def test_fwd_f32_small(layout):
    w = _small_workload(layout, True, 64, dtype="f32", seed=11)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        for mm in (ca.RA_MERGE_FUSED, ca.RA_MERGE_SEPARATE):
            say(f"fwd f32 layout={layout} rank={rank} merge={mm}")
            _, _, _, out, lse = _run_fwd(w, glob, rank, mm)
            _check_fwd(w, glob, rank, out, lse)


def test_tiny_fp32_all_ranks():
    """batch 1, 2 heads, d 64, N 512 over D = 4 simulated ranks, fp32
    N(0,1)*0.1, non-causal basic ring: every rank's out + lse against full
    softmax attention."""
    w = synth.WORKLOADS["tiny_fp32"]
    glob = synth.draw_global(w)
    outs = []
    for rank in range(w.world):
        say(f"tiny fp32 rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank)
        _check_fwd(w, glob, rank, out, lse)
        outs.append(out)
    full, _ = oracle.rank_share_forward(glob["q"], glob["k"], glob["v"], ca.BASIC, 1, 0, False)
    assert np.abs(np.concatenate(outs, axis=1) - full).max() <= 1e-4


@pytest.mark.parametrize("S", [1, 63, 64, 65, 129])
def test_fwd_edge_shapes(S):
    """One-row shards, exact and ragged tile boundaries."""
    for layout in (ca.BASIC, ca.ZIGZAG, ca.STRIPE):
        if layout == ca.ZIGZAG and S % 2:
            continue
        w = _small_workload(layout, True, 128, D=3, S=S, B=1, Hq=2, Hkv=1, seed=S)
        glob = synth.draw_global(w)
        for rank in range(w.world):
            say(f"edge S={S} layout={layout} rank={rank}")
            _, _, _, out, lse = _run_fwd(w, glob, rank)
            _check_fwd(w, glob, rank, out, lse)


def test_fwd_world_one_is_plain_attention():
    w = _small_workload(ca.BASIC, True, 128, D=1, S=300, seed=5)
    glob = synth.draw_global(w)
    say("world=1")
    _, _, _, out, lse = _run_fwd(w, glob, 0)
    _check_fwd(w, glob, 0, out, lse)


def test_fwd_is_deterministic():
    w = _small_workload(ca.ZIGZAG, True, 128, seed=9)
    glob = synth.draw_global(w)
    say("determinism")
    _, _, _, o1, l1 = _run_fwd(w, glob, 1)
    _, _, _, o2, l2 = _run_fwd(w, glob, 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_identity_v_gives_exact_zeros_where_masked():
    """V = identity over the keys (head_dim >= keys): out is the probability
    matrix, exactly zero on masked keys."""
    N, D, d = 128, 2, 128
    w = synth.Workload("eye", 1, 1, 1, d, N, D, 0, True, ca.STRIPE, "bf16", seed=3)
    glob = synth.draw_global(w)
    glob["v"] = np.zeros_like(glob["v"])
    glob["v"][0, :, 0, :N] = np.eye(N, dtype=np.float32)
    for rank in range(D):
        say(f"identity V rank={rank}")
        sh, desc, _, out, lse = _run_fwd(w, glob, rank)
        m = oracle.allowed(sh["pos_q"], np.arange(N), True)
        P = out[0, :, 0, :N]
        assert np.all(P[~m] == 0.0)
        assert np.all(P[m] > 0.0)


@pytest.mark.parametrize("d", [128, 64, 96, 4, 12, 260, 512])
def test_lse_merge_kernel(d):
    """Every head_dim the entry point accepts (multiples of 4), including rows
    that do not fill a power-of-two lane group (96, 12) and rows longer than
    one wave's 64 float4 items (260, 512)."""
    rng = np.random.default_rng(17 + d)
    B, S, H = 2, 777, 3
    o = rng.standard_normal((B, S, H, d)).astype(np.float32)
    oj = rng.standard_normal((B, S, H, d)).astype(np.float32)
    l = (rng.standard_normal((B, H, S)) * 5).astype(np.float32)
    lj = (rng.standard_normal((B, H, S)) * 5).astype(np.float32)
    l[0, 0, :10] = -np.inf            # empty running rows
    lj[0, 1, 5:20] = -np.inf          # empty partial rows
    l[1, 2, 30:40] = -np.inf
    lj[1, 2, 30:40] = -np.inf         # both empty
    o[0, :10, 0] = 0.0
    oj[0, 5:20, 1] = 0.0
    o[1, 30:40, 2] = 0.0
    oj[1, 30:40, 2] = 0.0
    say(f"lse merge d={d}")
    to = torch.from_numpy(o).cuda()
    tl = torch.from_numpy(l).cuda()
    ca.ring_attn_lse_merge(to, tl, torch.from_numpy(oj).cuda(), torch.from_numpy(lj).cuda())
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge(o.transpose(0, 2, 1, 3), l, oj.transpose(0, 2, 1, 3), lj)
    got_o = to.cpu().numpy().transpose(0, 2, 1, 3)
    assert np.abs(got_o - ref_o).max() < 1e-5
    assert max_err_lse(tl.cpu().numpy(), ref_l) < 1e-5
    assert not np.isnan(got_o).any()


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _check_bwd(w, glob, rank, dq, dk, dv):
    sh = shard(glob, w, rank)
    rdq, rdk, rdv = oracle.rank_share_backward(glob["q"], glob["k"], glob["v"], sh["dout"], w.layout,
                                               w.world, rank, w.causal, w.cu_seqlens,
                                               window=w.window)
    errs = {}
    scale = max(float(np.abs(r).max()) for r in (rdq, rdk, rdv))
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        e = float(np.abs(got - ref).max())
        bound = 5e-2 * float(np.abs(ref).max())
        if bound == 0.0:
            # exactly zero in exact arithmetic (a one-key window makes every
            # dS = P (dP - Delta) cancel): only fp32 rounding of that
            # difference may remain
            bound = 1e-4 * scale
        errs[name] = (e, bound)
        assert e <= bound, (name, e, bound)
    return errs


def _run_bwd(w, glob, rank, dk=None, dv=None, ds_store=True, ds_kv_heads=None):
    """Backward through the C ABI; ds_store=False gives it the minimum
    workspace, so that dQ recomputes S and dP instead of reading stored dS;
    ds_kv_heads=n gives it a dS store for n kv heads at a time."""
    sh = shard(glob, w, rank)
    desc = ca.desc_from_workload(w, rank=rank)
    q, k, v = (to_dev(sh[n], w.dtype) for n in ("q", "k", "v"))
    out, lse = ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens)
    dout = to_dev(sh["dout"], w.dtype)
    if ds_kv_heads is None:
        ws = ca.alloc_workspace(desc, True, cu_seqlens=w.cu_seqlens, ds_store=ds_store)
    else:
        per = -(-ca.ring_attn_bwd_ds_bytes(desc, w.cu_seqlens) // w.heads_kv)
        ws = torch.empty(ca.ring_attn_workspace_bytes(desc, True) + ds_kv_heads * per,
                         dtype=torch.uint8, device="cuda")
    dq, dk, dv = ca.ring_attn_bwd(desc, dout, q, k, v, out, lse, w.cu_seqlens, dk=dk, dv=dv,
                                  workspace=ws)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("ds_store", [True, False])
def test_bwd_is_deterministic(ds_store):
    """No kernel of the backward uses atomics: two calls on the same inputs
    give the same bits (dK/dV accumulated into zeroed buffers), for both dQ
    paths."""
    w = _small_workload(ca.ZIGZAG, True, 128, D=3, S=600, B=1, seed=11, with_grad=True)
    glob = synth.draw_global(w)
    say(f"bwd determinism ds_store={ds_store}")
    r1 = _run_bwd(w, glob, 1, ds_store=ds_store)
    r2 = _run_bwd(w, glob, 1, ds_store=ds_store)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("head_dim", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_small(layout, head_dim, causal):
    w = _small_workload(layout, causal, head_dim, seed=20 + layout, with_grad=True)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"bwd layout={layout} d={head_dim} causal={causal} rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank)
        _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("layout,head_dim,causal", [
    (ca.BASIC, 128, True), (ca.BASIC, 64, False), (ca.ZIGZAG, 128, True), (ca.STRIPE, 128, True),
    (ca.VARLEN_RING, 128, True), (ca.VARLEN_ZIGZAG, 128, True), (ca.VARLEN_STRIPE, 64, True)])
def test_bwd_several_tiles(layout, head_dim, causal):
    """Shards of 600 rows: three 256-row dQ tiles (the last ragged), five
    128-row forward tiles, ten 64-row dK/dV query tiles over 128-key tiles with
    a ragged last block, GQA 4/2."""
    w = _small_workload(layout, causal, head_dim, D=3, S=600, B=1, seed=40 + layout,
                        with_grad=True)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"bwd several tiles layout={layout} d={head_dim} causal={causal} rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank)
        _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


# ---------------------------------------------------------------------------
# Sliding windows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal,window", [(True, (70, -1)), (False, (45, 90)), (True, (0, -1))])
def test_fwd_window(layout, causal, window):
    """Sliding-window forward (bf16, d 128) on every layout; the basic layout
    with a narrow window leaves whole ring steps without a visible pair."""
    w = _small_workload(layout, causal, 128, seed=60 + layout, window=window)
    glob = synth.draw_global(w)
    for rank in (0, 1, w.world - 1):
        say(f"fwd window layout={layout} causal={causal} window={window} rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank)
        _check_fwd(w, glob, rank, out, lse)


def test_fwd_window_f32_separate_merge():
    w = _small_workload(ca.STRIPE, True, 64, dtype="f32", seed=66, window=(33, -1))
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"fwd window f32 separate rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank, ca.RA_MERGE_SEPARATE)
        _check_fwd(w, glob, rank, out, lse)


@pytest.mark.parametrize("layout,head_dim,causal,window", [
    (ca.BASIC, 128, True, (150, -1)), (ca.ZIGZAG, 128, True, (300, -1)),
    (ca.STRIPE, 64, False, (90, 60)), (ca.LLAMA3, 128, True, (200, -1)),
    (ca.VARLEN_ZIGZAG, 128, False, (-1, 100)), (ca.BASIC, 128, True, (0, -1))])
def test_bwd_window(layout, head_dim, causal, window):
    """Sliding-window backward on 600-row shards (several tiles, ragged tail)."""
    w = _small_workload(layout, causal, head_dim, D=3, S=600, B=1, seed=70 + layout,
                        with_grad=True, window=window)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"bwd window layout={layout} d={head_dim} causal={causal} window={window} rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank)
        _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("layout,head_dim,causal,window", [
    (ca.BASIC, 128, True, (-1, -1)), (ca.ZIGZAG, 64, True, (-1, -1)),
    (ca.LLAMA3, 128, True, (-1, -1)), (ca.STRIPE, 128, False, (80, 40))])
def test_bwd_recompute_path(layout, head_dim, causal, window):
    """With only the minimum workspace the dQ kernel recomputes S and dP; both
    backward paths meet the oracle on the same 600-row shards."""
    w = _small_workload(layout, causal, head_dim, D=3, S=600, B=1, seed=80 + layout,
                        with_grad=True, window=window)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"bwd recompute path layout={layout} d={head_dim} causal={causal} rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank, ds_store=False)
        _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())
        say(f"bwd stored-dS path layout={layout} d={head_dim} causal={causal} rank={rank}")
        dq2, dk2, dv2 = _run_bwd(w, glob, rank, ds_store=True)
        _check_bwd(w, glob, rank, dq2.cpu().numpy(), dk2.cpu().numpy(), dv2.cpu().numpy())


@pytest.mark.parametrize("S", [1, 63, 64, 65, 257])
def test_bwd_edge_shapes(S):
    """Backward on one-row shards and at exact and ragged tile boundaries
    (64-row dK/dV query tiles, 128-key tiles, 256-row dQ tiles), both dQ
    paths."""
    for layout in (ca.BASIC, ca.ZIGZAG, ca.STRIPE):
        if layout == ca.ZIGZAG and S % 2:
            continue
        w = _small_workload(layout, True, 128, D=3, S=S, B=1, Hq=2, Hkv=1, seed=S + 3,
                            with_grad=True)
        glob = synth.draw_global(w)
        for rank in range(w.world):
            for ds_store in (True, False):
                say(f"bwd edge S={S} layout={layout} rank={rank} ds_store={ds_store}")
                dq, dk, dv = _run_bwd(w, glob, rank, ds_store=ds_store)
                _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("layout,Hq,Hkv,ds_kv_heads", [
    (ca.BASIC, 6, 3, 1), (ca.BASIC, 6, 3, 2), (ca.ZIGZAG, 8, 4, 3), (ca.LLAMA3, 4, 4, 1),
    (ca.VARLEN_STRIPE, 6, 3, 2)])
def test_bwd_ds_store_in_kv_head_passes(layout, Hq, Hkv, ds_kv_heads):
    """A dS store for fewer kv heads than the problem has: the backward runs
    the kv heads in passes (the last one shorter when they do not divide)."""
    w = _small_workload(layout, True, 128, D=3, S=300, B=1, Hq=Hq, Hkv=Hkv, seed=90 + layout,
                        with_grad=True)
    glob = synth.draw_global(w)
    for rank in (0, w.world - 1):
        say(f"bwd kv-head passes layout={layout} Hq={Hq} Hkv={Hkv} per pass={ds_kv_heads} rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank, ds_kv_heads=ds_kv_heads)
        _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


def test_bwd_ranks_sum_to_full_gradient():
    """dk/dv accumulated over every rank's backward on the same buffers equal
    the full-sequence gradient; the ranks' dq tile the full dq."""
    w = _small_workload(ca.ZIGZAG, True, 128, D=4, S=160, B=1, seed=31, with_grad=True)
    glob = synth.draw_global(w)
    dk = dv = None
    dq_full = np.zeros_like(glob["q"])
    for rank in range(w.world):
        say(f"bwd sum over ranks rank={rank}")
        dq, dk, dv = _run_bwd(w, glob, rank, dk=dk, dv=dv)
        dq_full[:, oracle.positions(w.layout, w.seqlen, w.world, rank)] = dq.cpu().numpy()
    rdq, rdk, rdv = oracle.rank_share_backward(glob["q"], glob["k"], glob["v"], glob["dout"],
                                               ca.BASIC, 1, 0, True)
    blocks = [oracle.kv_positions(w.layout, w.seqlen, w.world, j) for j in range(w.world)]
    order = np.concatenate(blocks)
    got_dk = np.concatenate(list(dk.cpu().numpy()), axis=1)
    got_dv = np.concatenate(list(dv.cpu().numpy()), axis=1)
    for got, ref in ((got_dk, rdk[0][:, order]), (got_dv, rdv[0][:, order]), (dq_full, rdq)):
        assert np.abs(got - ref).max() <= 5e-2 * np.abs(ref).max()


def _random_config(seed):
    rng = np.random.default_rng(1000 + seed)
    layout = int(rng.choice(LAYOUTS))
    D = int(rng.choice([1, 2, 3, 4, 5, 8]))
    S = int(rng.integers(1, 700))
    if layout in (ca.ZIGZAG, ca.VARLEN_ZIGZAG) and S % 2:
        S += 1
    Hkv = int(rng.choice([1, 2, 3]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    window = [(-1, -1), (int(rng.integers(0, 300)), -1), (int(rng.integers(0, 200)), int(rng.integers(0, 200)))][
        int(rng.integers(0, 3))]
    N = D * S
    cu = None
    B = int(rng.choice([1, 2]))
    if layout in synth.VARLEN_LAYOUTS:
        m = synth.doc_multiple(layout, D)
        n_docs = int(rng.integers(1, max(2, min(6, N // m))))
        cu = tuple(synth.random_cu_seqlens(N, n_docs, rng, multiple=m))
        B = 1
    return synth.Workload(f"rand{seed}", B, Hq, Hkv, d, N, D, 0, causal, layout, "bf16",
                          seed=2000 + seed, cu_seqlens=cu, with_grad=True, window=window)


@pytest.mark.parametrize("seed", range(12))
def test_random_configs_fwd_f32(seed):
    """The fp32 forward (both merge modes) on seeded random configurations."""
    w = _random_config(100 + seed).replace(dtype="f32", with_grad=False, value_scale=0.5)
    glob = synth.draw_global(w)
    for rank in sorted({0, w.world - 1}):
        for mm in (ca.RA_MERGE_FUSED, ca.RA_MERGE_SEPARATE):
            say(f"random f32 seed={seed} layout={w.layout} D={w.world} S={w.shard} d={w.head_dim} "
                f"window={w.window} rank={rank} merge={mm}")
            _, _, _, out, lse = _run_fwd(w, glob, rank, mm)
            _check_fwd(w, glob, rank, out, lse)


@pytest.mark.parametrize("seed", range(24))
def test_random_configs_fwd_bwd(seed):
    """Seeded random shapes: layout, world, shard length, GQA ratio, head dim,
    causal flag, window, batch and document split; forward and both backward
    paths against the oracle for the first and last rank."""
    w = _random_config(seed)
    glob = synth.draw_global(w)
    for rank in sorted({0, w.world - 1}):
        say(f"random seed={seed} layout={w.layout} D={w.world} S={w.shard} B={w.batch} "
            f"Hq={w.heads_q} Hkv={w.heads_kv} d={w.head_dim} causal={w.causal} window={w.window} "
            f"rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank)
        _check_fwd(w, glob, rank, out, lse)
        for ds_store in (True, False):
            dq, dk, dv = _run_bwd(w, glob, rank, ds_store=ds_store)
            _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("Hq,Hkv,layout", [(8, 1, ca.BASIC), (16, 2, ca.VARLEN_RING),
                                            (32, 1, ca.ZIGZAG), (12, 4, ca.STRIPE)])
def test_gqa_large_groups(Hq, Hkv, layout):
    """Query-head groups larger than the random configurations draw (up to 32
    q heads on one kv head): the forward reads kv head h * Hkv / Hq, the
    dK/dV kernel walks every q head of its group, both dQ paths."""
    w = _small_workload(layout, True, 64, D=2, S=264, B=1, Hq=Hq, Hkv=Hkv, seed=Hq + Hkv,
                        with_grad=True)
    glob = synth.draw_global(w)
    for rank in range(w.world):
        say(f"gqa Hq={Hq} Hkv={Hkv} layout={layout} rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank)
        _check_fwd(w, glob, rank, out, lse)
        for ds_store in (True, False):
            dq, dk, dv = _run_bwd(w, glob, rank, ds_store=ds_store)
            _check_bwd(w, glob, rank, dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy())


@pytest.mark.parametrize("layout,B,head_dim,S", [(ca.ZIGZAG, 2, 64, 1250), (ca.LLAMA3, 1, 128, 2300),
                                                 (ca.BASIC, 2, 128, 1100)])
def test_fwd_persistent_schedule(layout, B, head_dim, S):
    """More work items (batch x q heads x 256-row query tiles) than CUs: the
    one-launch forward runs one work-group per CU, each walking the planner's
    list of items (lists of unequal length, ragged last tile), and must give
    the oracle's result on every row."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # the same token geometry with two head counts (and head dims): each call
    # needs the schedule of its own (batch, q head) pairs
    for Hq, d in ((32, head_dim), (40, 192 - head_dim)):
        w = _small_workload(layout, True, d, D=2, S=S, B=B, Hq=Hq, Hkv=8, seed=S + layout)
        assert w.batch * w.heads_q * -(-S // 256) > cus
        glob = synth.draw_global(w)
        for rank in range(w.world):
            say(f"persistent forward layout={layout} B={w.batch} Hq={Hq} d={d} S={S} rank={rank}")
            _, _, _, out, lse = _run_fwd(w, glob, rank)
            _check_fwd(w, glob, rank, out, lse)


@pytest.mark.parametrize("layout,causal,window,head_dim,S,B,Hq", [
    (ca.STRIPE, True, (-1, -1), 128, 1100, 2, 32),
    (ca.VARLEN_ZIGZAG, True, (-1, -1), 64, 1800, 1, 40),
    (ca.VARLEN_STRIPE, False, (-1, -1), 128, 1200, 1, 64),
    (ca.BASIC, True, (700, -1), 128, 1100, 2, 32),
    (ca.VARLEN_RING, False, (300, 200), 64, 1500, 1, 48)])
def test_fwd_persistent_schedule_layouts(layout, causal, window, head_dim, S, B, Hq):
    """The persistent forward on the other layouts, without the causal mask
    and with sliding windows (masked tiles at both ends of a list, steps with
    no visible pair), more work items than CUs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = _small_workload(layout, causal, head_dim, D=2, S=S, B=B, Hq=Hq, Hkv=8, seed=S + 11 * layout,
                        window=window)
    assert w.batch * w.heads_q * -(-S // 256) > cus
    glob = synth.draw_global(w)
    for rank in range(w.world):
        say(f"persistent forward layout={layout} causal={causal} window={window} d={head_dim} "
            f"S={S} B={w.batch} Hq={Hq} rank={rank}")
        _, _, _, out, lse = _run_fwd(w, glob, rank)
        _check_fwd(w, glob, rank, out, lse)


@pytest.mark.parametrize("layout,B,head_dim,S", [(ca.LLAMA3, 1, 128, 2300), (ca.LLAMA3, 1, 64, 2300)])
def test_fwd_split_lists(layout, B, head_dim, S):
    """Packed documents of very different lengths give query-tile lists of
    very different lengths: with the part buffer in the workspace the
    persistent forward cuts the longest lists into parts on different CUs and
    merges them (the part-merge kernel runs); without it the lists run whole.
    Both match the oracle, and differ from each other only by the rounding of
    the merge."""
    _split_against_whole(_small_workload(layout, True, head_dim, D=2, S=S, B=B, Hq=32, Hkv=8,
                                         seed=3 * S + layout))


def test_fwd_split_lists_across_ring_steps():
    """A varlen ring share whose lists hold the key tiles of four ring steps:
    eight short documents and a long one give lists of very different
    lengths (the planner's cost model cuts this share, checked below through
    the part-merge launches), and the cuts of the long lists fall inside and
    between ring steps (each part walks entries of several steps, with their
    blocks and key intervals)."""
    cu = (0, 344, 688, 1032, 1376, 1720, 2064, 2408, 2768, 9216)
    w = synth.Workload("split-varlen-ring", 1, 32, 8, 128, 9216, 4, 0, True, ca.VARLEN_RING, "bf16",
                       seed=77, cu_seqlens=cu)
    _split_against_whole(w)


def _split_against_whole(w):
    glob = synth.draw_global(w)
    rank = w.world - 1
    layout, head_dim, S = w.layout, w.head_dim, w.shard
    sh = shard(glob, w, rank)
    desc = ca.desc_from_workload(w, rank=rank)
    q, k, v = (to_dev(sh[n], w.dtype) for n in ("q", "k", "v"))
    split_bytes = ca.ring_attn_fwd_split_bytes(desc)
    assert split_bytes > 0
    ref = oracle.rank_share_forward(glob["q"], glob["k"], glob["v"], w.layout, w.world, rank, w.causal,
                                    w.cu_seqlens, window=w.window)
    results = {}
    for name, nbytes in (("split", ca.ring_attn_workspace_bytes(desc, False) + split_bytes),
                         ("whole", 16)):
        say(f"split lists layout={layout} d={head_dim} S={S} workspace={name}")
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ca.ring_attn_timing_enable(False)
        ca.ring_attn_timing_enable(True)
        out, lse = ca.ring_attn_fwd(desc, q, k, v, w.cu_seqlens, workspace=ws)
        torch.cuda.synchronize()
        merges, _ = ca.ring_attn_timing_read("fwd_part_merge")
        ca.ring_attn_timing_enable(False)
        assert (merges > 0) == (name == "split"), (name, merges)
        results[name] = (out.float().cpu().numpy(), lse.cpu().numpy())
        _check_fwd(w, glob, rank, *results[name], ref=ref)
    assert np.abs(results["split"][0] - results["whole"][0]).max() <= 1e-2
    assert max_err_lse(results["split"][1], results["whole"][1]) <= 1e-4


def test_hip_graph_capture_and_replay():
    """After a first eager call (which builds the plan), the forward and the
    backward enqueue only kernels: they can be captured into a HIP graph.  The
    graph is replayed several times, with other work and synchronisations in
    between, and every replay must reproduce the eager results exactly."""
    w = _small_workload(ca.ZIGZAG, True, 128, D=4, S=320, B=1, seed=123, with_grad=True)
    glob = synth.draw_global(w)
    sh = shard(glob, w, 1)
    desc = ca.desc_from_workload(w, rank=1)
    q, k, v = (to_dev(sh[n], w.dtype) for n in ("q", "k", "v"))
    dout = to_dev(sh["dout"], w.dtype)
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads_q, w.shard, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(v.shape, dtype=torch.float32, device="cuda")
    ws_f = ca.alloc_workspace(desc, False)
    ws_b = ca.alloc_workspace(desc, True)

    def run(stream=None):
        dk.zero_()   # a fill kernel, not a memset node
        dv.zero_()
        ca.ring_attn_fwd(desc, q, k, v, None, out, lse, ws_f, stream=stream)
        ca.ring_attn_bwd(desc, dout, q, k, v, out, lse, None, dq, dk, dv, ws_b, stream=stream)

    say("graph: eager reference")
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, lse, dq, dk, dv):   # eager work between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            assert torch.equal(got, want), (rep, name)
    _check_fwd(w, glob, 1, out.float().cpu().numpy(), lse.cpu().numpy())


def test_no_plan_is_built_during_capture():
    """Building a plan allocates and uploads, which a graph cannot hold: a call
    for a shape that was never planned, made while its stream is captured,
    returns RA_E_NO_PLAN before enqueuing anything; after an eager call has
    planned the shape, the same call captures and replays correctly."""
    w = _small_workload(ca.STRIPE, True, 64, D=4, S=136, B=1, seed=321)
    glob = synth.draw_global(w)
    sh = shard(glob, w, 2)
    desc = ca.desc_from_workload(w, rank=2)
    q, k, v = (to_dev(sh[n], w.dtype) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    lse = torch.empty(w.batch, w.heads_q, w.shard, device="cuda")
    ca.ring_attn_clear_cache()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    say("capture: unplanned shape")
    err = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out.zero_()   # a fill kernel, so that the graph is not empty
            try:
                ca.ring_attn_fwd(desc, q, k, v, None, out, lse, stream=s)
            except ca.RingAttnError as e:
                err = e
    torch.cuda.synchronize()
    assert err is not None and err.code == -12, err
    n, _ = ca.ring_attn_plan_cache_info()
    assert n == 0
    say("capture: after an eager call")
    ca.ring_attn_fwd(desc, q, k, v, None, out, lse)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    g2 = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g2, stream=s):
            ca.ring_attn_fwd(desc, q, k, v, None, out, lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(2):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), rep


def test_plan_cache_is_bounded():
    """Packed training sends new document boundaries every step: 200 forward
    calls with distinct cu_seqlens keep at most the cache limit of plans, and
    once the cache is full the library's device memory stays the same."""
    D, S, H, d = 4, 96, 2, 64
    N = D * S
    rng = np.random.default_rng(404)
    q = torch.randn(1, S, H, d, device="cuda").to(torch.bfloat16)
    k = torch.randn(D, 1, S, H, d, device="cuda").to(torch.bfloat16)
    v = torch.randn(D, 1, S, H, d, device="cuda").to(torch.bfloat16)
    ca.ring_attn_clear_cache()
    prev = ca.ring_attn_plan_cache_limit(8)
    try:
        seen, used = set(), []
        say("plan cache: 200 calls with distinct cu_seqlens")
        while len(seen) < 200:
            cu = tuple(synth.random_cu_seqlens(N, 5, rng, multiple=D))
            if cu in seen:
                continue
            seen.add(cu)
            desc = ca.make_desc(1, H, H, d, N, D, 1, True, ca.VARLEN_RING, cu_seqlens=cu)
            ca.ring_attn_fwd(desc, q, k, v, cu)
            n, nbytes = ca.ring_attn_plan_cache_info()
            assert n == min(len(seen), 8)
            used.append((nbytes, torch.cuda.mem_get_info()[0]))
        torch.cuda.synchronize()
        # plans of this shape differ only in their tile lists (a few KiB): the
        # bytes held stay below 8 of the largest, and the device's free memory
        # stops moving once the cache is full
        largest = max(used[0][0], *(b - a for (a, _), (b, _) in zip(used[:7], used[1:8])))
        assert max(b for b, _ in used) <= 8 * largest
        free = [f for _, f in used[20:]]
        assert max(free) - min(free) <= 4 << 20, (max(free), min(free))
    finally:
        ca.ring_attn_plan_cache_limit(prev)
        ca.ring_attn_clear_cache()
