"""Shared test plumbing: shard seeded global tensors for one rank using the
oracle's position maps (test infrastructure), and move them to the device."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from context_attention_flash_amd import synth


def say(msg: str):
    """Name the case on stdout (flushed) before any GPU work."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def shard(glob: dict, w: synth.Workload, rank: int):
    """q (and dout) rows of `rank` in local order; k, v block-major."""
    cu = list(w.cu_seqlens) if w.cu_seqlens is not None else None
    pos_q = oracle.positions(w.layout, w.seqlen, w.world, rank, cu)
    nb = oracle.num_blocks(w.layout, w.world)
    blocks = [oracle.kv_positions(w.layout, w.seqlen, w.world, j, cu) for j in range(nb)]
    res = {
        "q": np.ascontiguousarray(glob["q"][:, pos_q]),
        "k": np.ascontiguousarray(np.stack([glob["k"][:, pk] for pk in blocks])),
        "v": np.ascontiguousarray(np.stack([glob["v"][:, pk] for pk in blocks])),
        "pos_q": pos_q,
        "blocks": blocks,
    }
    if "dout" in glob:
        res["dout"] = np.ascontiguousarray(glob["dout"][:, pos_q])
    return res


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def tol(dtype: str):
    """Tolerances: fp32 out and lse <= 1e-4; bf16 out <= 2e-2, lse <= 1e-3;
    gradients <= 5e-2 of the oracle's max |grad| per tensor."""
    if dtype == "f32":
        return dict(out=1e-4, lse=1e-4)
    return dict(out=2e-2, lse=1e-3)


def max_err_lse(got: np.ndarray, ref: np.ndarray) -> float:
    """Max |lse error|; -inf must match -inf exactly."""
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "lse -inf pattern differs"
    if not fin.any():
        return 0.0
    return float(np.abs(got[fin] - ref[fin]).max())
