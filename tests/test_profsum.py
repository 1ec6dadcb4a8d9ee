"""Host-side checks of the rocprofv3 summary reader used by bench.py."""
from context_attention_flash_amd import profsum


def _write(tmp_path, kernel, digest, value):
    p = tmp_path / "t.md"
    p.write_text(f"# x\n\n```\nkernel: {kernel}\nkernel_source_sha256_16: {digest}\n"
                 f"traffic_bytes_per_launch: {value}\n```\n")
    return str(p)


def test_traffic_read_only_while_sources_match(tmp_path):
    k = "bwd_dkdv_bf16_kernel"
    good = _write(tmp_path, k, profsum.source_hash(k), "1.5e+09")
    assert profsum.read_traffic(good, k) == 1.5e9
    assert profsum.read_traffic(good, "fwd_step_bf16_kernel") is None      # another kernel
    stale = _write(tmp_path, k, "0" * 16, "1.5e+09")
    assert profsum.read_traffic(stale, k) is None                          # sources changed
    assert profsum.read_traffic(str(tmp_path / "missing.md"), k) is None


def test_committed_summary_parses():
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = os.path.join(root, "profiles", "traffic_bwd_dkdv_bf16_kernel_basic_s8192.md")
    kv = {}
    for line in open(p):
        if ": " in line and line.strip().split(": ")[0].replace("_", "").isalnum():
            a, b = line.strip().split(": ", 1)
            kv[a] = b
    assert kv["kernel"] == "bwd_dkdv_bf16_kernel"
    assert float(kv["traffic_bytes_per_launch"]) > 0
