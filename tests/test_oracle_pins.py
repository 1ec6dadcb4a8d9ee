"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the passage or the mathematical fact it checks:
  * the two-device worked example of the ai360xpert "Ring Attention" page
    ("Show Me the Code"): ring == single-device attention to ~1e-15;
  * exactness of the ring decomposition for every D and layout (same page,
    "Online softmax across ring steps"; zenaique "same exact math");
  * the causal rule "step <= rank" (instagit/nanotron "Forward Pass
    Implementation");
  * brute force with explicit loops and math.fsum;
  * closed forms (Q = 0 gives the mean of the visible values and
    lse = ln(#visible); V = const; V = identity gives the probability matrix);
  * central finite differences for the gradients;
  * torch's fp64 scaled_dot_product_attention with an explicit boolean mask and
    autograd (an independent library routine).
A few tests plant a mistake in a copy of the oracle and check that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BASIC, ZIGZAG, STRIPE, VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE, PACKED
from context_attention_flash_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [BASIC, ZIGZAG, STRIPE, VARLEN_RING, LLAMA3, VARLEN_ZIGZAG, VARLEN_STRIPE]


def _cu_for(layout, n, world, rng):
    if layout == LLAMA3:
        return synth.random_cu_seqlens(n, 4, rng)
    if layout in PACKED:
        m = synth.doc_multiple(layout, world)
        return synth.random_cu_seqlens(n, min(3, n // m), rng, multiple=m)
    return None


def _inputs(rng, B, N, Hq, Hkv, d, scale=1.0):
    q = rng.standard_normal((B, N, Hq, d)) * scale
    k = rng.standard_normal((B, N, Hkv, d)) * scale
    v = rng.standard_normal((B, N, Hkv, d)) * scale
    return q, k, v


# ---------------------------------------------------------------------------
# The pages' worked example
# ---------------------------------------------------------------------------

def _two_device_example():
    with open(os.path.join(GOLDEN, "ra_two_device_example.json")) as f:
        g = json.load(f)
    r = g["recipe"]
    rng = np.random.default_rng(r["seed"])
    n, d = r["n"], r["d"]
    Q = rng.standard_normal((n, d)) * 0.1
    K = rng.standard_normal((n, d)) * 0.1
    V = rng.standard_normal((n, d)) * 0.1
    return g, Q[None, :, None, :], K[None, :, None, :], V[None, :, None, :]


def _ring_vs_plain_two_devices(mod):
    g, Q, K, V = _two_device_example()
    D = g["recipe"]["devices"]
    ring = np.concatenate([mod.ring_forward(Q, K, V, BASIC, D, r, False)[0] for r in range(D)], axis=1)
    plain, _ = oracle.rank_share_forward(Q, K, V, BASIC, 1, 0, False)
    return g, np.abs(ring - plain).max()


def test_pages_two_device_example():
    g, err = _ring_vs_plain_two_devices(oracle)
    assert err <= g["pin_tolerance"], err


def test_planted_merge_without_rescale_fails_example(monkeypatch):
    """A merge that averages partials without the LSE weights must fail the
    pages' example (the pin would catch a dropped term in the merge)."""
    import oracle.ring_oracle as ro

    def bad_merge(out, lse, out_j, lse_j):
        return 0.5 * (out + out_j), np.logaddexp(lse, lse_j)

    monkeypatch.setattr(ro, "lse_merge", bad_merge)
    g, err = _ring_vs_plain_two_devices(ro)
    assert err > 100 * g["pin_tolerance"]


def test_planted_sign_error_in_merge_fails_example(monkeypatch):
    import oracle.ring_oracle as ro
    good = ro.lse_merge

    def bad_merge(out, lse, out_j, lse_j):
        o, l = good(out, lse, out_j, -lse_j)
        return o, l

    monkeypatch.setattr(ro, "lse_merge", bad_merge)
    g, err = _ring_vs_plain_two_devices(ro)
    assert err > 100 * g["pin_tolerance"]


# ---------------------------------------------------------------------------
# torch fp64 SDPA + autograd (independent library routine)
# ---------------------------------------------------------------------------

def _sdpa_reference(q, k, v, dout_local, layout, world, rank, causal, cu, window=(-1, -1)):
    """Full-sequence attention by torch SDPA in fp64 with an explicit mask,
    restricted to the rank's rows; gradients by autograd."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    cu_l = cu if layout in PACKED else None
    pos_q = oracle.positions(layout, N, world, rank, cu_l)
    # mask from the definition on global positions, written out here directly
    t = np.arange(N)
    mask = np.ones((N, N), bool)
    if causal:
        mask &= t[None, :] <= t[:, None]
    if cu_l is not None:
        doc = np.zeros(N, np.int64)
        for i, (a, b) in enumerate(zip(cu_l[:-1], cu_l[1:])):
            doc[a:b] = i
        mask &= doc[None, :] == doc[:, None]
    for i in range(N):  # sliding window, row by row
        if window[0] >= 0:
            mask[i, :max(0, i - window[0])] = False
        if window[1] >= 0:
            mask[i, i + window[1] + 1:] = False
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    g = Hq // Hkv
    qh = qt.permute(0, 2, 1, 3)
    kh = kt.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vh = vt.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    out = torch.nn.functional.scaled_dot_product_attention(
        qh, kh, vh, attn_mask=torch.tensor(mask), scale=1.0 / math.sqrt(d))
    out = out.permute(0, 2, 1, 3)  # [B, N, Hq, d]
    out_rank = out[:, torch.tensor(pos_q)]
    res = {"out": out_rank.detach().numpy()}
    if dout_local is not None:
        (out_rank * torch.tensor(dout_local)).sum().backward()
        res["dq"] = qt.grad[:, torch.tensor(pos_q)].numpy()
        nb = oracle.num_blocks(layout, world)
        blocks = [oracle.kv_positions(layout, N, world, j, cu_l) for j in range(nb)]
        res["dk"] = np.stack([kt.grad.numpy()[:, pk] for pk in blocks])
        res["dv"] = np.stack([vt.grad.numpy()[:, pk] for pk in blocks])
    return res


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_forward_and_grads_match_torch_sdpa(layout, causal):
    rng = np.random.default_rng(100 + layout * 2 + causal)
    world, B, Hq, Hkv, d = 4, 2, 4, 2, 8
    N = 48
    if layout in PACKED:
        B = 1
    cu = _cu_for(layout, N, world, rng)
    q, k, v = _inputs(rng, B, N, Hq, Hkv, d)
    for rank in range(world):
        S = len(oracle.positions(layout, N, world, rank, cu))
        dout = rng.standard_normal((B, S, Hq, d))
        ref = _sdpa_reference(q, k, v, dout, layout, world, rank, causal, cu)
        out, lse = oracle.rank_share_forward(q, k, v, layout, world, rank, causal, cu)
        assert np.abs(out - ref["out"]).max() < 1e-12
        dq, dk, dv = oracle.rank_share_backward(q, k, v, dout, layout, world, rank, causal, cu)
        assert np.abs(dq - ref["dq"]).max() < 1e-11
        assert np.abs(dk - ref["dk"]).max() < 1e-11
        assert np.abs(dv - ref["dv"]).max() < 1e-11


def test_d1_reduces_to_plain_attention():
    rng = np.random.default_rng(7)
    q, k, v = _inputs(rng, 2, 40, 2, 2, 16)
    for causal in (True, False):
        ref = _sdpa_reference(q, k, v, None, BASIC, 1, 0, causal, None)
        ring, _ = oracle.ring_forward(q, k, v, BASIC, 1, 0, causal)
        assert np.abs(ring - ref["out"]).max() < 1e-12


# ---------------------------------------------------------------------------
# Ring decomposition == unblocked attention (exactness)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_ring_equals_unblocked(layout, world, causal):
    rng = np.random.default_rng(1000 + 10 * layout + world + 100 * causal)
    N = 2 * world * 5
    B = 1 if layout in PACKED else 2
    if layout == VARLEN_RING and N // world < 3:
        N = world * 6
    cu = _cu_for(layout, N, world, rng)
    q, k, v = _inputs(rng, B, N, 4, 2, 8)
    for rank in range(world):
        a, la = oracle.rank_share_forward(q, k, v, layout, world, rank, causal, cu)
        b, lb = oracle.ring_forward(q, k, v, layout, world, rank, causal, cu)
        assert np.abs(a - b).max() < 1e-12
        fin = np.isfinite(la)
        assert np.array_equal(fin, np.isfinite(lb))
        assert np.abs(la[fin] - lb[fin]).max() < 1e-12


def test_causal_rank_share_with_skipped_steps_is_restricted_full_causal():
    """instagit "Forward Pass Implementation": only steps with step <= rank are
    computed under a causal mask; the result must equal full causal attention
    restricted to the rank's rows."""
    rng = np.random.default_rng(11)
    N, D = 64, 4
    q, k, v = _inputs(rng, 2, N, 2, 2, 8)
    full = _sdpa_reference(q, k, v, None, BASIC, 1, 0, True, None)["out"]
    S = N // D
    for r in range(D):
        parts = []
        ring, _ = oracle.ring_forward(q, k, v, BASIC, D, r, True, partial_out=parts)
        assert [p[0] for p in parts] == list(range(r + 1))
        assert [p[1] for p in parts] == [(r - s) % D for s in range(r + 1)]
        assert np.abs(ring - full[:, r * S:(r + 1) * S]).max() < 1e-12


def test_ring_order():
    assert oracle.ring_schedule(4, 1) == [(0, 1), (1, 0), (2, 3), (3, 2)]


# ---------------------------------------------------------------------------
# The packed ring layout (VARLEN_RING): rank -> part map and the step rule
# ---------------------------------------------------------------------------

# Written out by hand from the layout's definition: documents [0, 8) and
# [8, 20) over D = 4 ranks have parts of 2 and 3 tokens; rank r holds part r of
# each document, in document order.
VARLEN_RING_LITERAL = {"cu": [0, 8, 20], "world": 4,
                       "ranks": [[0, 1, 8, 9, 10], [2, 3, 11, 12, 13],
                                 [4, 5, 14, 15, 16], [6, 7, 17, 18, 19]]}


def _varlen_ring_pin_failures(mod):
    """Every failed check of the packed ring layout against facts the pages fix
    (instagit/nanotron "Forward Pass Implementation": the varlen forward runs
    a step only when step <= rank under a causal mask; skillfed "ring-flash-
    attn": every variant comes in a varlen form that shares one cu_seqlens for
    q and kv).  Returns a list of strings; empty when the oracle passes."""
    bad = []
    L = VARLEN_RING_LITERAL
    for r, want in enumerate(L["ranks"]):
        got = mod.positions(VARLEN_RING, L["cu"][-1], L["world"], r, L["cu"]).tolist()
        if got != want:
            bad.append(f"literal rank {r}: {got} != {want}")
    # Causal pair counts per step, per document of length L_k (part P = L_k/D):
    # a block that precedes the rank's part in every document is fully visible
    # (P^2 pairs), the rank's own part is a causal triangle (P(P+1)/2), and a
    # later block is invisible; so exactly the steps s <= rank are active.
    D = 4
    cu = [0, 8, 20, 44, 48]   # lengths 8, 12, 24, 4: parts 2, 3, 6, 1
    parts = np.diff(cu) // D
    for r in range(D):
        counts = mod.step_pair_counts(VARLEN_RING, cu[-1], D, r, True, cu)
        for s, j, pairs in counts:
            want = int((parts ** 2).sum() if j < r else
                       (parts * (parts + 1) // 2).sum() if j == r else 0)
            if pairs != want:
                bad.append(f"rank {r} step {s} block {j}: {pairs} pairs != {want}")
        active = [s for s, _, p in counts if p > 0]
        if active != list(range(r + 1)):
            bad.append(f"rank {r}: active steps {active} != step <= rank")
    # The causal rank share with the steps s > rank skipped equals full
    # per-document causal attention (plain definition, written out here over
    # the whole packed stream) restricted to the rank's rows.
    rng = np.random.default_rng(31)
    N = cu[-1]
    q, k, v = _inputs(rng, 1, N, 2, 2, 8)
    t = np.arange(N)
    doc = np.searchsorted(np.asarray(cu), t, side="right") - 1
    mask = (t[None, :] <= t[:, None]) & (doc[None, :] == doc[:, None])
    sc = np.einsum("thd,uhd->htu", q[0], k[0]) / math.sqrt(8)
    sc = np.where(mask[None], sc, -np.inf)
    p = np.exp(sc - sc.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    full = np.einsum("htu,uhd->thd", p, v[0])
    for r in range(D):
        rows = mod.positions(VARLEN_RING, N, D, r, cu)
        parts_seen = []
        ring, _ = mod.ring_forward(q, k, v, VARLEN_RING, D, r, True, cu, partial_out=parts_seen)
        kept = [(s, j, o, l) for s, j, o, l in parts_seen if s <= r]
        o_run, l_run = kept[0][2], kept[0][3]
        for _, _, o, l in kept[1:]:
            o_run, l_run = mod.lse_merge(o_run, l_run, o, l)
        skipped = np.transpose(o_run, (0, 2, 1, 3))[0]
        if np.abs(skipped - full[rows]).max() > 1e-12 or np.abs(ring[0] - full[rows]).max() > 1e-12:
            bad.append(f"rank {r}: rank share with steps s > rank skipped != causal attention")
    return bad


def test_varlen_ring_layout_and_step_rule():
    assert _varlen_ring_pin_failures(oracle) == []


@pytest.mark.parametrize("plant", ["reversed_parts", "interleaved_parts"])
def test_planted_varlen_ring_map_fails(plant, monkeypatch):
    """A rank-reversed part map (rank r holds part D-1-r) or an in-document
    interleave (rank r holds tokens a + r + D*i) must fail the pins above."""
    import oracle.ring_oracle as ro
    good = ro.positions

    def bad_positions(layout, n, world, rank, cu_seqlens=None):
        if layout != VARLEN_RING:
            return good(layout, n, world, rank, cu_seqlens)
        parts = []
        for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
            part = (b - a) // world
            if plant == "reversed_parts":
                parts.append(a + (world - 1 - rank) * part + np.arange(part, dtype=np.int64))
            else:
                parts.append(a + rank + world * np.arange(part, dtype=np.int64))
        return np.concatenate(parts)

    monkeypatch.setattr(ro, "positions", bad_positions)
    assert len(_varlen_ring_pin_failures(ro)) > 0


# ---------------------------------------------------------------------------
# Brute force with explicit loops
# ---------------------------------------------------------------------------

def _brute(q, k, v, pos_q, causal, cu, scale):
    """Explicit loops with math.fsum: out/lse of each row over all global keys."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    out = np.zeros((B, len(pos_q), Hq, d))
    lse = np.zeros((B, Hq, len(pos_q)))

    def doc(t):
        if cu is None:
            return 0
        for i in range(len(cu) - 1):
            if cu[i] <= t < cu[i + 1]:
                return i
        raise AssertionError

    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i, t in enumerate(pos_q):
                keys = [u for u in range(N) if (not causal or u <= t) and doc(u) == doc(t)]
                if not keys:
                    lse[b, h, i] = -math.inf
                    continue
                sc = [scale * math.fsum(float(q[b, t, h, c]) * float(k[b, u, hk, c]) for c in range(d))
                      for u in keys]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                tot = math.fsum(e)
                lse[b, h, i] = m + math.log(tot)
                for c in range(d):
                    out[b, i, h, c] = math.fsum(e[j] * float(v[b, u, hk, c]) for j, u in enumerate(keys)) / tot
    return out, lse


@pytest.mark.parametrize("layout", LAYOUTS)
def test_brute_force_tiny(layout):
    rng = np.random.default_rng(55 + layout)
    N, D = 16, 2
    B = 1
    cu = _cu_for(layout, N, D, rng)
    q, k, v = _inputs(rng, B, N, 2, 1, 4)
    for causal in (True, False):
        for r in range(D):
            cu_l = cu if layout in PACKED else None
            pos_q = oracle.positions(layout, N, D, r, cu_l)
            bo, bl = _brute(q, k, v, pos_q, causal, cu_l, 0.5)
            o, l = oracle.rank_share_forward(q, k, v, layout, D, r, causal, cu, scale=0.5)
            o2, l2 = oracle.ring_forward(q, k, v, layout, D, r, causal, cu, scale=0.5)
            assert np.abs(o - bo).max() < 1e-13 and np.abs(o2 - bo).max() < 1e-13
            assert np.abs(l - bl).max() < 1e-13 and np.abs(l2 - bl).max() < 1e-13


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [(-1, -1), (5, -1), (3, 2), (-1, 4)])
def test_zero_query_gives_mean_and_log_count(layout, causal, window):
    """Q = 0: every visible score is 0, so out_t = mean of the visible v_u and
    lse_t = ln(#visible_t).  The visible keys are the interval from
    max(doc_start, t - left) to min(t, doc_end - 1, t + right) (the causal and
    window bounds only where they apply); doc_start = 0, doc_end = N in batch
    mode."""
    rng = np.random.default_rng(77 + layout)
    N, D = 32, 4
    B = 1 if layout in PACKED else 2
    cu = _cu_for(layout, N, D, rng)
    cu_l = cu if layout in PACKED else None
    q, k, v = _inputs(rng, B, N, 2, 2, 8)
    q[:] = 0.0
    for r in range(D):
        pos_q = oracle.positions(layout, N, D, r, cu_l)
        o, l = oracle.ring_forward(q, k, v, layout, D, r, causal, cu, window=window)
        for i, t in enumerate(pos_q):
            if cu_l is None:
                start, end = 0, N
            else:
                di = int(np.searchsorted(cu_l, t, side="right") - 1)
                start, end = cu_l[di], cu_l[di + 1]
            hi = t + 1 if causal else end
            if window[0] >= 0:
                start = max(start, t - window[0])
            if window[1] >= 0:
                hi = min(hi, t + window[1] + 1)
            cnt = hi - start
            assert np.allclose(l[:, :, i], math.log(cnt), atol=1e-13, rtol=0)
            for h in range(2):
                assert np.allclose(o[:, i, h], v[:, start:hi, h].mean(axis=1), atol=1e-13, rtol=0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_window_of_one_token_is_the_token_itself(layout):
    """A window (0, 0) (or left 0 under the causal mask) leaves each query only
    its own key: out_t = v_t and lse_t = scale <q_t, k_t>, for every rank."""
    rng = np.random.default_rng(91 + layout)
    N, D, d = 48, 4, 8
    B = 1 if layout in PACKED else 2
    cu = _cu_for(layout, N, D, rng)
    cu_l = cu if layout in PACKED else None
    q, k, v = _inputs(rng, B, N, 4, 2, d)
    for causal, window in ((True, (0, -1)), (False, (0, 0)), (True, (0, 7))):
        for r in range(D):
            pos_q = oracle.positions(layout, N, D, r, cu_l)
            o, l = oracle.ring_forward(q, k, v, layout, D, r, causal, cu, window=window)
            o2, l2 = oracle.rank_share_forward(q, k, v, layout, D, r, causal, cu, window=window)
            for h in range(4):
                hk = h // 2
                assert np.abs(o[:, :, h] - v[:, pos_q, hk]).max() < 1e-14
                assert np.abs(o2[:, :, h] - v[:, pos_q, hk]).max() < 1e-14
                dots = (q[:, pos_q, h] * k[:, pos_q, hk]).sum(-1) / math.sqrt(d)
                assert np.abs(l[:, h] - dots).max() < 1e-13
                assert np.abs(l2[:, h] - dots).max() < 1e-13


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal,window", [(True, (6, -1)), (False, (5, 3)), (False, (-1, 2))])
def test_window_matches_torch_sdpa_and_ring(layout, causal, window):
    """Windowed rank shares against torch fp64 SDPA with the window mask built
    row by row in the test, forward and gradients; the ring decomposition
    matches as well; a window wider than the sequence is plain attention."""
    rng = np.random.default_rng(300 + layout * 3 + causal)
    world, N, d = 4, 48, 8
    B = 1 if layout in PACKED else 2
    cu = _cu_for(layout, N, world, rng)
    q, k, v = _inputs(rng, B, N, 4, 2, d)
    for rank in range(world):
        S = len(oracle.positions(layout, N, world, rank, cu if layout in PACKED else None))
        dout = rng.standard_normal((B, S, 4, d))
        ref = _sdpa_reference(q, k, v, dout, layout, world, rank, causal, cu, window)
        out, lse = oracle.rank_share_forward(q, k, v, layout, world, rank, causal, cu, window=window)
        assert np.abs(out - ref["out"]).max() < 1e-12
        ring, lr = oracle.ring_forward(q, k, v, layout, world, rank, causal, cu, window=window)
        assert np.abs(ring - out).max() < 1e-12 and np.abs(lr - lse).max() < 1e-12
        dq, dk, dv = oracle.rank_share_backward(q, k, v, dout, layout, world, rank, causal, cu,
                                                window=window)
        assert np.abs(dq - ref["dq"]).max() < 1e-11
        assert np.abs(dk - ref["dk"]).max() < 1e-11
        assert np.abs(dv - ref["dv"]).max() < 1e-11
        wide, _ = oracle.rank_share_forward(q, k, v, layout, world, rank, causal, cu,
                                            window=(N, N))
        plain, _ = oracle.rank_share_forward(q, k, v, layout, world, rank, causal, cu)
        assert np.array_equal(wide, plain)


def test_constant_v_and_rows_sum_to_one():
    rng = np.random.default_rng(3)
    for layout in LAYOUTS:
        N, D = 24, 3 if layout != ZIGZAG else 2
        B = 1
        cu = _cu_for(layout, N, D, rng)
        q, k, v = _inputs(rng, B, N, 2, 2, 8, scale=3.0)
        v[:] = 1.0
        v[..., 3] = -2.5
        for r in range(D):
            o, _ = oracle.ring_forward(q, k, v, layout, D, r, True, cu)
            assert np.abs(o[..., :3] - 1.0).max() < 1e-13
            assert np.abs(o[..., 3] + 2.5).max() < 1e-13


@pytest.mark.parametrize("layout", LAYOUTS)
def test_identity_v_gives_probability_matrix(layout):
    """V = identity over the keys: out row t is the probability vector of row t;
    it is exactly zero on masked keys and sums to one."""
    rng = np.random.default_rng(21 + layout)
    N, D = 16, 2
    cu = _cu_for(layout, N, D, rng)
    cu_l = cu if layout in PACKED else None
    q = rng.standard_normal((1, N, 1, N))
    k = rng.standard_normal((1, N, 1, N))
    v = np.eye(N)[None, :, None, :]
    for r in range(D):
        pos_q = oracle.positions(layout, N, D, r, cu_l)
        o, _ = oracle.ring_forward(q, k, v, layout, D, r, True, cu)
        P = o[0, :, 0, :]
        for i, t in enumerate(pos_q):
            for u in range(N):
                same_doc = cu_l is None or np.searchsorted(cu_l, u, "right") == np.searchsorted(cu_l, t, "right")
                if u > t or not same_doc:
                    assert P[i, u] == 0.0
                else:
                    assert P[i, u] > 0.0
        assert np.abs(P.sum(axis=1) - 1.0).max() < 1e-13


def test_merge_identities():
    rng = np.random.default_rng(9)
    o = rng.standard_normal((5, 7))
    l = rng.standard_normal(5)
    # identical partials: same out, lse + ln 2
    mo, ml = oracle.lse_merge(o, l, o, l)
    assert np.abs(mo - o).max() < 1e-14 and np.abs(ml - (l + math.log(2))).max() < 1e-14
    # an empty partial (lse = -inf) is the identity, on either side
    e = np.full(5, -np.inf)
    mo, ml = oracle.lse_merge(o, l, np.zeros_like(o), e)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(np.zeros_like(o), e, o, l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    # two empty partials stay empty without NaN
    mo, ml = oracle.lse_merge(np.zeros_like(o), e, np.zeros_like(o), e)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # huge lse values do not overflow (the bound is a few ulps of 800 ~ 1.1e-13,
    # the rounding of lse itself at that magnitude)
    mo, ml = oracle.lse_merge(o, l + 800.0, 2 * o, l + 800.0)
    assert np.abs(mo - 1.5 * o).max() < 1e-12


# ---------------------------------------------------------------------------
# Gradients
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [BASIC, ZIGZAG, STRIPE, LLAMA3])
def test_gradients_by_central_differences(layout):
    rng = np.random.default_rng(31 + layout)
    N, D, r = 16, 2, 1
    B = 1
    cu = _cu_for(layout, N, D, rng)
    q, k, v = _inputs(rng, B, N, 2, 1, 4)
    S = len(oracle.positions(layout, N, D, r, cu if layout in PACKED else None))
    dout = rng.standard_normal((B, S, 2, 4))
    dq, dk, dv = oracle.rank_share_backward(q, k, v, dout, layout, D, r, True, cu)
    nb = oracle.num_blocks(layout, D)
    blocks = [oracle.kv_positions(layout, N, D, j, cu if layout in PACKED else None)
              for j in range(nb)]
    cu_l = cu if layout in PACKED else None
    pos_q = oracle.positions(layout, N, D, r, cu_l)

    def loss(q_, k_, v_):
        o, _ = oracle.rank_share_forward(q_, k_, v_, layout, D, r, True, cu)
        return float((o * dout).sum())

    h = 1e-5
    for _ in range(12):
        which = rng.integers(3)
        arr = [q, k, v][which]
        idx = tuple(int(rng.integers(s)) for s in arr.shape)
        plus = [x.copy() for x in (q, k, v)]
        minus = [x.copy() for x in (q, k, v)]
        plus[which][idx] += h
        minus[which][idx] -= h
        fd = (loss(*plus) - loss(*minus)) / (2 * h)
        b, t, hh, c = idx
        if which == 0:
            loc = np.nonzero(pos_q == t)[0]
            an = dq[b, loc[0], hh, c] if len(loc) else 0.0
        else:
            g = dk if which == 1 else dv
            an = 0.0
            for j, pk in enumerate(blocks):
                loc = np.nonzero(pk == t)[0]
                if len(loc):
                    an = g[j, b, loc[0], hh, c]
        assert abs(fd - an) < 1e-7, (which, idx, fd, an)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_rank_gradients_sum_to_full_gradient(layout):
    """instagit "Backward Pass and Gradient Accumulation": dk/dv of a block are
    the sum of every rank's contribution; dq of the ranks tile the full dq."""
    rng = np.random.default_rng(41 + layout)
    N, D = 24, 3 if layout != ZIGZAG else 2
    N = 24
    cu = _cu_for(layout, N, D, rng)
    cu_l = cu if layout in PACKED else None
    q, k, v = _inputs(rng, 1, N, 4, 2, 8)
    dout_g = rng.standard_normal((1, N, 4, 8))
    full = _sdpa_reference(q, k, v, dout_g, BASIC if cu_l is None else LLAMA3, 1, 0, True, cu)
    dk_sum = None
    dq_full = np.zeros_like(q)
    for r in range(D):
        pos_q = oracle.positions(layout, N, D, r, cu_l)
        dq, dk, dv = oracle.rank_share_backward(q, k, v, dout_g[:, pos_q], layout, D, r, True, cu)
        dq_full[:, pos_q] = dq
        dk_sum = dk if dk_sum is None else dk_sum + dk
        dv_sum = dv if r == 0 else dv_sum + dv
    nb = oracle.num_blocks(layout, D)
    blocks = [oracle.kv_positions(layout, N, D, j, cu_l) for j in range(nb)]
    full_dk = np.concatenate([dk_sum[j] for j in range(nb)], axis=1)
    full_dv = np.concatenate([dv_sum[j] for j in range(nb)], axis=1)
    order = np.concatenate(blocks)
    assert np.abs(full_dk - full["dk"][0][:, order]).max() < 1e-11
    assert np.abs(full_dv - full["dv"][0][:, order]).max() < 1e-11
    assert np.abs(dq_full - full["dq"]).max() < 1e-11


# ---------------------------------------------------------------------------
# Layout facts
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("world", [1, 2, 3, 4, 8])
def test_layout_is_a_bijection(layout, world):
    rng = np.random.default_rng(5)
    N = 2 * world * 6
    cu = _cu_for(layout, N, world, rng)
    cu_l = cu if layout in PACKED else None
    allpos = np.concatenate([oracle.positions(layout, N, world, r, cu_l) for r in range(world)])
    assert np.array_equal(np.sort(allpos), np.arange(N))
    for r in range(world):
        p = oracle.positions(layout, N, world, r, cu_l)
        assert len(p) == N // world
        assert np.all(np.diff(p) > 0)  # local order is increasing global order


def test_zigzag_and_stripe_pair_counts():
    N, D = 64, 4
    c = N // (2 * D)
    S = N // D
    for r in range(D):
        counts = oracle.step_pair_counts(ZIGZAG, N, D, r, True)
        for s, j, pairs in counts:
            assert pairs == (2 * c * c + c if s == 0 else 2 * c * c)
        counts = oracle.step_pair_counts(STRIPE, N, D, r, True)
        for s, j, pairs in counts:
            assert pairs == (S * (S + 1) // 2 if j <= r else S * (S - 1) // 2)
        counts = oracle.step_pair_counts(BASIC, N, D, r, True)
        for s, j, pairs in counts:
            assert pairs == (S * (S + 1) // 2 if s == 0 else (S * S if s <= r else 0))


def test_varlen_zigzag_and_stripe_pair_counts():
    """Documents never see each other, so the packed forms' causal pair counts
    are the per-document closed forms of ZIGZAG / STRIPE summed over the
    documents; every rank also holds exactly L/D tokens of each document."""
    D = 4
    cu = [0, 8, 40, 64, 128]  # document lengths 8, 32, 24, 64: multiples of 2D
    N = cu[-1]
    lens = np.diff(cu)
    for r in range(D):
        for layout in (VARLEN_ZIGZAG, VARLEN_STRIPE):
            p = oracle.positions(layout, N, D, r, cu)
            per_doc = np.histogram(p, bins=cu)[0]
            assert np.array_equal(per_doc, lens // D)
        for s, j, pairs in oracle.step_pair_counts(VARLEN_ZIGZAG, N, D, r, True, cu):
            c = lens // (2 * D)
            assert pairs == int((2 * c * c + (c if s == 0 else 0)).sum())
        for s, j, pairs in oracle.step_pair_counts(VARLEN_STRIPE, N, D, r, True, cu):
            Sk = lens // D
            assert pairs == int((Sk * (Sk + 1) // 2 if j <= r else Sk * (Sk - 1) // 2).sum())
    # a single document is the batch form
    for r in range(D):
        assert np.array_equal(oracle.positions(VARLEN_ZIGZAG, N, D, r, [0, N]),
                              oracle.positions(ZIGZAG, N, D, r))
        assert np.array_equal(oracle.positions(VARLEN_STRIPE, N, D, r, [0, N]),
                              oracle.positions(STRIPE, N, D, r))


def test_workload_pair_totals():
    """Visible pairs of the benchmark workloads, from closed forms:
    basic causal rank r of D: r*S^2 + S(S+1)/2; zigzag: 16c^2 + c at D = 8;
    llama3: sum over the rank's rows of (t - doc_start + 1)."""
    w = synth.WORKLOADS["basic_s4096"]
    S = w.shard
    tot = sum(p for _, _, p in oracle.step_pair_counts(BASIC, w.seqlen, w.world, w.rank, True))
    assert tot == 7 * S * S + S * (S + 1) // 2 == 125_831_168
    w = synth.WORKLOADS["llama3"]
    cu = list(w.cu_seqlens)
    tot = oracle.step_pair_counts(LLAMA3, w.seqlen, w.world, w.rank, True, cu)[0][2]
    S = w.shard
    expect = 0
    for t in range(w.rank * S, (w.rank + 1) * S):
        di = max(i for i in range(len(cu) - 1) if cu[i] <= t)
        expect += t - cu[di] + 1
    assert tot == expect == 88_502_272


def test_llama3_cu_seqlens_recipe():
    cu = synth.lognormal_cu_seqlens(65536, 2048, 1.0, 64, 16384, np.random.default_rng(2004))
    if np.__version__.startswith("2.2"):
        assert cu == synth.LLAMA3_CU_SEQLENS
    assert synth.LLAMA3_CU_SEQLENS[-1] == 65536


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0, 1.0 + 2 ** -9, 65504.0], np.float32)
    q = synth.quantize_bf16(x)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(q, ref)
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    assert np.array_equal(synth.quantize_bf16(r), torch.tensor(r).to(torch.bfloat16).float().numpy())


def test_backward_key_range_is_exact_and_guarded():
    """Restricting the backward's sums to a key range that holds every visible
    key changes nothing (invisible keys carry weight 0); a range that drops a
    visible key is refused."""
    rng = np.random.default_rng(77)
    N, D, r = 96, 4, 2
    cu = [0, 10, 40, 70, 96]
    q, k, v = _inputs(rng, 1, N, 4, 2, 8)
    S = N // D
    dout = rng.standard_normal((1, S, 4, 8))
    full = oracle.rank_share_backward(q, k, v, dout, LLAMA3, D, r, True, cu)
    # rank 2 holds [48, 72): documents [40, 70) and [70, 96) -> keys [40, 72)
    part = oracle.rank_share_backward(q, k, v, dout, LLAMA3, D, r, True, cu, key_range=(40, 72))
    for a, b in zip(full, part):
        assert np.abs(a - b).max() < 1e-12
    with pytest.raises(ValueError):
        oracle.rank_share_backward(q, k, v, dout, LLAMA3, D, r, True, cu, key_range=(41, 72))
