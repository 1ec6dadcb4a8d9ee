"""Argument checks of the autograd wrapper, on the host: unsupported options
are refused, and host tensors are rejected (there is no CPU path)."""
import pytest

torch = pytest.importorskip("torch")

import context_attention_flash_amd as ca  # noqa: E402
from context_attention_flash_amd.autograd import (ring_flash_attn_func,  # noqa: E402
                                                  ring_flash_attn_varlen_func)


def _qkv(B=1, S=64, H=2, d=64, D=2, dtype=torch.bfloat16):
    q = torch.zeros(B, S, H, d, dtype=dtype)
    k = torch.zeros(D, B, S, H, d, dtype=dtype)
    return q, k, k.clone()


def test_refuses_unsupported_options():
    q, k, v = _qkv()
    with pytest.raises(NotImplementedError, match="dropout"):
        ring_flash_attn_func(q, k, v, dropout_p=0.1, world=2)
    with pytest.raises(NotImplementedError, match="alibi"):
        ring_flash_attn_func(q, k, v, alibi_slopes=torch.ones(2), world=2)
    with pytest.raises(ValueError, match="window_size"):
        ring_flash_attn_func(q, k, v, window_size=(-2, 0), world=2)
    with pytest.raises(ValueError, match="packed layouts"):
        ring_flash_attn_func(q, k, v, world=2, layout=ca.VARLEN_RING)
    with pytest.raises(ValueError, match="batch layouts"):
        ring_flash_attn_varlen_func(q[0], k[:, 0], v[:, 0], [0, 128], world=2, layout=ca.ZIGZAG)
    with pytest.raises(ValueError, match="cu_seqlens ends"):
        ring_flash_attn_varlen_func(q[0], k[:, 0], v[:, 0], [0, 64], world=2)


def test_host_tensors_are_rejected_not_computed():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="device tensor"):
        ring_flash_attn_func(q, k, v, causal=True, world=2, rank=1)
    with pytest.raises(ValueError, match="device tensor"):
        ring_flash_attn_varlen_func(q[0], k[:, 0], v[:, 0], [0, 32, 128], causal=True, world=2,
                                    rank=0)
