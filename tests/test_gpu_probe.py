"""The measurement probes bench.py uses: the streaming copy, add and
read-only fold compute exactly what they claim over the bytes they are given
(the unrolled passes and the tail, every cache policy), so their bandwidths
are those of correct kernels; the MFMA-only kernels run and write finite
sums."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _probe():
    lib = ctypes.CDLL(os.path.join(ROOT, "context_attention_flash_amd", "libraprobe.so"))
    lib.ra_probe_stream.restype = ctypes.c_int
    lib.ra_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.ra_probe_stream_read.restype = ctypes.c_int
    lib.ra_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("flags", [0, 3])
@pytest.mark.parametrize("chunks, blocks", [(1, 1), (100003, 7), (1 << 22, 2048), (3 * 256 * 8 + 5, 3)])
def test_stream_is_exact(chunks, blocks, flags, add):
    import torch
    lib = _probe()
    g = torch.Generator(device="cuda")
    g.manual_seed(chunks + 7 * flags + add)
    a = torch.randn(chunks * 4, device="cuda", generator=g)
    b = torch.randn(chunks * 4, device="cuda", generator=g)
    dst = torch.full((chunks * 4 + 4,), 7.0, device="cuda")   # one guard chunk past the end
    print("stream", "add" if add else "copy", chunks, "chunks,", blocks, "blocks, flags", flags,
          flush=True)
    rc = lib.ra_probe_stream(a.data_ptr(), b.data_ptr() if add else None, dst.data_ptr(), chunks * 16,
                             blocks, flags, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(dst[: chunks * 4], a + b if add else a)
    assert torch.equal(dst[chunks * 4:], torch.full((4,), 7.0, device="cuda"))


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("chunks, blocks", [(1, 1), (100003, 7), (1 << 22, 2048), (3 * 256 * 8 + 5, 3)])
def test_stream_read_visits_every_word_once(chunks, blocks, flags):
    """Every thread folds its chunks with xor, so the xor of all the threads'
    words is the xor of every 32-bit word read, each exactly once."""
    import numpy as np
    import torch
    lib = _probe()
    g = torch.Generator(device="cuda")
    g.manual_seed(chunks + 7 * flags)
    a = torch.randint(-2**31, 2**31 - 1, (chunks * 4,), dtype=torch.int32, device="cuda", generator=g)
    out = torch.full((blocks * 256 + 1,), 12345, dtype=torch.int32, device="cuda")  # one guard word
    print("stream read", chunks, "chunks,", blocks, "blocks, flags", flags, flush=True)
    rc = lib.ra_probe_stream_read(a.data_ptr(), out.data_ptr(), chunks * 16, blocks, flags,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out[:-1].cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(a.cpu().numpy().view(np.uint32))
    assert got == want
    assert int(out[-1]) == 12345


@pytest.mark.parametrize("random_operands", [False, True])
def test_mfma_probes_run_and_give_finite_sums(random_operands):
    """The MFMA-only kernels the bench times: every lane writes a finite,
    non-zero sum of its accumulators (a launch that did no MFMA would leave
    the sentinel)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "context_attention_flash_amd", "libraprobe.so"))
    fn = lib.ra_probe_mfma_random if random_operands else lib.ra_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    blocks = 16
    out = torch.full((blocks * 256,), float("nan"), device="cuda")
    print("mfma probe, random operands" if random_operands else "mfma probe", flush=True)
    assert fn(out.data_ptr(), blocks, 64, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    assert (out != 0).any().item()
