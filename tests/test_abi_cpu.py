"""Host-side checks of the C ABI (no GPU needed, no device work enqueued).

* the library loads and exports every entry point include/ring_attn.h declares;
* position maps and ring schedules are bit-exact against the oracle for every
  layout, world size, rank and document split;
* tile classification agrees with a brute-force element mask;
* every validation error is returned before any device call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import context_attention_flash_amd as ca
import oracle
from context_attention_flash_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LAYOUTS = [ca.BASIC, ca.ZIGZAG, ca.STRIPE, ca.VARLEN_RING, ca.LLAMA3, ca.VARLEN_ZIGZAG,
           ca.VARLEN_STRIPE]


def test_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "ring_attn.h")).read()
    declared = set(re.findall(r"\b(ring_attn_\w+)\s*\(", header))
    assert len(declared) >= 13
    lib = ca.lib()
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert ca.ring_attn_version() == 1


def test_peak_probe_library_loads():
    """bench.py's probes are built beside the library and export their calls;
    the MFMA probe's flop count is the kernel's (4 waves x 4 chains x 32x32x16x2
    per MFMA, the MFMAs per chain rounded up to a multiple of 8); the streaming
    probe refuses null or misaligned pointers, sizes that are not a multiple of
    16 bytes, empty grids and unknown flags."""
    lib = ctypes.CDLL(os.path.join(ROOT, "context_attention_flash_amd", "libraprobe.so"))
    assert hasattr(lib, "ra_probe_mfma")
    lib.ra_probe_mfma_flops.restype = ctypes.c_double
    lib.ra_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    assert lib.ra_probe_mfma_flops(2, 8) == 2 * 4 * 8 * 4 * 32768.0
    assert lib.ra_probe_mfma_flops(1, 9) == 4 * 16 * 4 * 32768.0
    lib.ra_probe_mfma.restype = ctypes.c_int
    lib.ra_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert lib.ra_probe_mfma(None, 1, 8, None) != 0   # refused before any launch
    lib.ra_probe_mfma_random.restype = ctypes.c_int
    lib.ra_probe_mfma_random.argtypes = lib.ra_probe_mfma.argtypes
    for out, blocks, iters in ((None, 1, 8), (16, 0, 8), (16, 1, 0)):
        assert lib.ra_probe_mfma_random(out, blocks, iters, None) != 0
    lib.ra_probe_stream.restype = ctypes.c_int
    lib.ra_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    for a, b, dst, nbytes, blocks, flags in (
            (None, None, 16, 16, 1, 0), (16, None, None, 16, 1, 0), (16, None, 32, 24, 1, 0),
            (16, None, 32, 16, 0, 0), (8, None, 32, 16, 1, 0), (16, 40, 32, 16, 1, 0),
            (16, None, 32, -16, 1, 0), (16, None, 32, 16, 1, 4), (16, None, 32, 16, 1, -1)):
        assert lib.ra_probe_stream(a, b, dst, nbytes, blocks, flags, None) != 0   # refused, no launch
    assert lib.ra_probe_stream(16, 48, 32, 0, 1, 3, None) == 0                   # nothing to move
    lib.ra_probe_stream_read.restype = ctypes.c_int
    lib.ra_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    for a, out, nbytes, blocks, flags in (
            (None, 16, 16, 1, 0), (16, None, 16, 1, 0), (16, 32, 24, 1, 0), (16, 32, 16, 0, 0),
            (8, 32, 16, 1, 0), (16, 40, 16, 1, 0), (16, 32, -16, 1, 0), (16, 32, 16, 1, 2),
            (16, 32, 16, 1, -1)):
        assert lib.ra_probe_stream_read(a, out, nbytes, blocks, flags, None) != 0  # refused
    assert lib.ra_probe_stream_read(16, 32, 0, 1, 1, None) == 0                 # nothing to read


def _cu(layout, N, D, rng, n_docs=5):
    if layout not in synth.VARLEN_LAYOUTS:
        return None
    m = synth.doc_multiple(layout, D)
    return synth.random_cu_seqlens(N, min(n_docs, N // m), rng, multiple=m)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("D", [1, 2, 3, 4, 8])
def test_positions_bit_exact(layout, D):
    rng = np.random.default_rng(D * 10 + layout)
    for N in (2 * D * 7, 2 * D * 64):
        cu = _cu(layout, N, D, rng)
        for r in range(D):
            desc = ca.make_desc(1, 2, 1, 128, N, D, r, True, layout, cu_seqlens=cu)
            cu_l = cu if layout in synth.VARLEN_LAYOUTS else None
            got = ca.ring_attn_positions(desc, cu)
            assert got.dtype == np.int64
            assert np.array_equal(got, oracle.positions(layout, N, D, r, cu_l))
            for j in range(oracle.num_blocks(layout, D)):
                assert np.array_equal(ca.ring_attn_kv_positions(desc, cu, j),
                                      oracle.kv_positions(layout, N, D, j, cu_l))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [(-1, -1), (17, -1), (9, 30), (-1, 5), (0, 0)])
def test_schedule_matches_oracle_pair_counts(layout, causal, window):
    rng = np.random.default_rng(3 + layout)
    for D in (1, 2, 4, 8):
        N = 2 * D * 24
        cu = _cu(layout, N, D, rng)
        for r in range(D):
            desc = ca.make_desc(2, 4, 2, 64, N, D, r, causal, layout, cu_seqlens=cu,
                                window=window)
            if cu is not None:
                desc.batch = 1
            got = ca.ring_attn_schedule(desc, cu)
            ref = oracle.step_pair_counts(layout, N, D, r, causal, cu, window)
            assert got == ref


def test_basic_causal_schedule_is_step_le_rank():
    """instagit "Forward Pass Implementation": under a causal mask only steps
    with step <= rank are computed."""
    D, N = 8, 8 * 32
    for r in range(D):
        desc = ca.make_desc(1, 1, 1, 128, N, D, r, True, ca.BASIC)
        for s, j, pairs in ca.ring_attn_schedule(desc):
            assert j == (r - s) % D
            assert (pairs > 0) == (s <= r)


def test_workload_pair_totals_from_library():
    for name, total in (("basic_s4096", 125_831_168), ("zigzag", 1_073_750_016),
                        ("llama3", 88_502_272), ("basic_s8192", 503_320_576)):
        w = synth.WORKLOADS[name]
        desc = ca.desc_from_workload(w)
        assert sum(p for _, _, p in ca.ring_attn_schedule(desc, w.cu_seqlens)) == total


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [(-1, -1), (21, 13)])
def test_tile_kinds_against_brute_force(layout, causal, window):
    rng = np.random.default_rng(50 + layout)
    for D, N, tq, tk in ((2, 2 * 2 * 45, 16, 8), (4, 4 * 2 * 40, 32, 16), (3, 3 * 2 * 30, 8, 32)):
        cu = _cu(layout, N, D, rng, n_docs=4)
        cu_l = cu if layout in synth.VARLEN_LAYOUTS else None
        for r in range(D):
            desc = ca.make_desc(1, 1, 1, 64, N, D, r, causal, layout, cu_seqlens=cu,
                                window=window)
            pos_q = oracle.positions(layout, N, D, r, cu_l)
            for s, j, _ in ca.ring_attn_schedule(desc, cu):
                pos_k = oracle.kv_positions(layout, N, D, j, cu_l)
                m = oracle.allowed(pos_q, pos_k, causal, cu_l, window)
                kinds = ca.ring_attn_tile_kinds(desc, cu, s, tq, tk)
                for qt in range(kinds.shape[0]):
                    for kt in range(kinds.shape[1]):
                        blk = m[qt * tq:(qt + 1) * tq, kt * tk:(kt + 1) * tk]
                        full_width = (kt + 1) * tk <= len(pos_k)
                        if kinds[qt, kt] == 2:
                            assert blk.all() and full_width
                        elif kinds[qt, kt] == 0:
                            assert not blk.any()
                        else:
                            assert blk.any() and not (blk.all() and full_width)


def test_fwd_split_bytes_without_device_work():
    """The split part buffer exists only for the one-launch bf16 forward: other
    dtypes and merge modes need none, and an unsupported head_dim or a null
    descriptor is refused, all without touching a device."""
    lib = ca.lib()
    d32 = ca.make_desc(1, 4, 2, 128, 64, 4, 1, True, ca.BASIC, dtype="f32")
    assert lib.ring_attn_fwd_split_bytes(ctypes.byref(d32)) == 0
    for mode in (ca.RA_MERGE_SEPARATE, ca.RA_MERGE_STEPWISE):
        d = ca.make_desc(1, 4, 2, 128, 64, 4, 1, True, ca.BASIC, merge_mode=mode)
        assert lib.ring_attn_fwd_split_bytes(ctypes.byref(d)) == 0
    bad = ca.make_desc(1, 4, 2, 96, 64, 4, 1, True, ca.BASIC)
    assert lib.ring_attn_fwd_split_bytes(ctypes.byref(bad)) < 0
    assert lib.ring_attn_fwd_split_bytes(None) < 0


def _rc_fwd(desc, cu=None, ws_bytes=1 << 30, nulls=False):
    """Calls ring_attn_fwd with fake non-null device pointers: validation must
    fail before any of them is touched."""
    fake = ctypes.c_void_p(0x1000) if not nulls else None
    keep, cup = ca._cu_arg(cu)
    return ca.lib().ring_attn_fwd(ctypes.byref(desc), fake, fake, fake, cup, fake, fake, fake,
                                  ws_bytes, None)


def test_validation_errors_before_device_work():
    ok = dict(batch=1, heads_q=4, heads_kv=2, head_dim=128, seqlen=64, world=4, rank=1,
              causal=True, layout=ca.BASIC)

    def d(**kw):
        a = dict(ok)
        a.update(kw)
        cu = a.pop("cu", None)
        return ca.make_desc(**a, cu_seqlens=cu), cu

    cases = [
        (dict(batch=0), -2), (dict(heads_q=0), -2), (dict(seqlen=0), -2),
        (dict(heads_q=3), -6), (dict(world=0), -3), (dict(rank=4), -3), (dict(rank=-1), -3),
        (dict(seqlen=66), -4), (dict(layout=ca.ZIGZAG, seqlen=68), -4), (dict(layout=7), -9),
        (dict(layout=ca.LLAMA3, batch=2, cu=[0, 64]), -9),
        (dict(layout=ca.LLAMA3, cu=[0, 10, 63]), -5), (dict(layout=ca.LLAMA3, cu=[1, 64]), -5),
        (dict(layout=ca.LLAMA3, cu=[0, 40, 30, 64]), -5),
        (dict(layout=ca.VARLEN_RING, cu=[0, 10, 64]), -5),
        (dict(layout=ca.VARLEN_ZIGZAG, cu=[0, 12, 64]), -5),
        (dict(layout=ca.VARLEN_ZIGZAG, cu=[0, 16, 64], seqlen=68), -4),
        (dict(layout=ca.VARLEN_STRIPE, cu=[0, 6, 64]), -5),
        (dict(layout=ca.VARLEN_STRIPE, batch=2, cu=[0, 64]), -9),
        (dict(head_dim=96), -7), (dict(dtype=5), -7),
        (dict(window=(-2, -1)), -11), (dict(window=(3, -5)), -11),
        (dict(softmax_scale=float("nan")), -11), (dict(softmax_scale=float("inf")), -11),
        (dict(softmax_scale=float("-inf")), -11),
    ]
    for kw, code in cases:
        desc, cu = d(**kw)
        assert _rc_fwd(desc, cu) == code, (kw, code)
        assert ca.ring_attn_strerror(code) != "unknown error code"
    desc, _ = d()
    assert _rc_fwd(desc, nulls=True) == -1
    desc.merge_mode = ca.RA_MERGE_STEPWISE   # the one-launch forward needs no workspace
    assert _rc_fwd(desc, ws_bytes=16) == -8
    desc.merge_mode = ca.RA_MERGE_SEPARATE
    assert _rc_fwd(desc, ws_bytes=16) == -8
    desc, _ = d(layout=ca.LLAMA3)
    desc.n_seqs = 1
    assert _rc_fwd(desc, None) == -1  # varlen without cu_seqlens
    # backward only has a bf16 kernel
    desc, _ = d(dtype="f32")
    fake = ctypes.c_void_p(0x1000)
    rc = ca.lib().ring_attn_bwd(ctypes.byref(desc), *([fake] * 6), None, fake, fake, fake, fake,
                                1 << 30, None)
    assert rc == -7
    # a NaN / infinite scale is refused by every entry point that reads the descriptor
    for bad in (float("nan"), float("inf")):
        desc, _ = d(softmax_scale=bad)
        assert ca.lib().ring_attn_workspace_bytes(ctypes.byref(desc), 0) == -11
        assert ca.lib().ring_attn_workspace_bytes(ctypes.byref(desc), 1) == -11
    # merge: bad head_dim
    assert ca.lib().ring_attn_lse_merge(fake, fake, fake, fake, 1, 4, 2, 6, None) == -2


def test_workspace_sizes():
    desc = ca.make_desc(1, 32, 32, 128, 32768, 8, 7, True, ca.BASIC)
    S_pad = 4096
    assert ca.ring_attn_workspace_bytes(desc, False) == 0   # one launch, registers
    desc.merge_mode = ca.RA_MERGE_STEPWISE
    assert ca.ring_attn_workspace_bytes(desc, False) == 32 * S_pad * 128 * 4
    desc.merge_mode = ca.RA_MERGE_FUSED
    desc.dtype = ca.RA_F32                                   # fp32: one launch per step
    assert ca.ring_attn_workspace_bytes(desc, False) == 32 * S_pad * 128 * 4
    desc.dtype = ca.RA_BF16
    assert ca.ring_attn_workspace_bytes(desc, True) == 2 * 32 * S_pad * 4 + 32 * S_pad * 128 * 4
    desc.merge_mode = ca.RA_MERGE_SEPARATE
    assert ca.ring_attn_workspace_bytes(desc, False) == 2 * 32 * 4096 * 128 * 4 + 32 * 4096 * 4
    desc.world = 0
    assert ca.lib().ring_attn_workspace_bytes(ctypes.byref(desc), 0) == -3
    with pytest.raises(ca.RingAttnError, match="RA_E_WORLD"):
        ca.ring_attn_workspace_bytes(desc, False)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ds_store_bytes_count_the_busiest_step(layout):
    """The dS tile store holds B * Hq * 16 KiB per non-empty 64 x 128 tile of
    the step with the most of them."""
    rng = np.random.default_rng(70 + layout)
    D, N = 4, 4 * 2 * 96
    cu = _cu(layout, N, D, rng)
    for causal in (True, False):
        for r in (0, D - 1):
            desc = ca.make_desc(1 if cu else 2, 4, 2, 128, N, D, r, causal, layout,
                                cu_seqlens=cu)
            most = 0
            for s, j, pairs in ca.ring_attn_schedule(desc, cu):
                if pairs:
                    most = max(most, int((ca.ring_attn_tile_kinds(desc, cu, s, 64, 128) > 0).sum()))
            assert ca.ring_attn_bwd_ds_bytes(desc, cu) == desc.batch * 4 * most * 64 * 128 * 2


def test_ds_store_bytes_basic_s4096():
    desc = ca.make_desc(1, 32, 32, 128, 32768, 8, 7, True, ca.BASIC)
    assert ca.ring_attn_bwd_ds_bytes(desc) == 32 * (4096 // 64) * (4096 // 128) * 16384


def test_python_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(ca, "_lib", None)
    monkeypatch.setattr(ca, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ca.lib()
