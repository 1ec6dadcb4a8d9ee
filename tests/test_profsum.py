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


def test_mfma_summary_from_counter_rows(tmp_path):
    """Per-kernel issued flops (MOPS x 512), busy fraction and clock from
    counter rows summed over the XCD instances of each dispatch."""
    import csv
    rows = []
    for d, name, mops, busy, gui in ((1, "void ra::fwd_step_bf16_kernel<128>(ra::FwdArgs)", 1000, 4096, 8000),
                                     (2, "ra::bwd_dkdv_bf16_kernel<128, true>(ra::BwdArgs)", 3000, 2048, 8000),
                                     (3, "void ra::bwd_dq_bf16_kernel<128>(ra::DqArgs)", 50, 512, 8000)):
            for xcd in range(8):   # one row per XCD instance
                for cname, val in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 8),
                                   ("SQ_VALU_MFMA_BUSY_CYCLES", busy / 8), ("GRBM_GUI_ACTIVE", gui / 8)):
                    rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": cname,
                                 "Counter_Value": val, "Start_Timestamp": 0, "End_Timestamp": 500})
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    md = profsum.mfma_md(str(p), "cmd", "title")
    out = tmp_path / "m.md"
    out.write_text(md)
    assert profsum.read_issued(str(out), "fwd_step_bf16_kernel") == 1000 * 512
    assert profsum.read_issued(str(out), "bwd_dkdv_bf16_kernel") == 3000 * 512
    assert profsum.read_issued(str(out), "bwd_dq_bf16_kernel") == 50 * 512
    assert profsum.read_issued(str(out), "bwd_dq_ds_bf16_kernel") is None   # not in the rows
    # busy = 4096 / (8000 / 8 * 1024) = 0.4%; clock = 8000 / 8 / 500 ns = 2.00 GHz
    assert "| `fwd_step_bf16_kernel` | 1 | 0.0 | 0.4% | 2.00 |" in md   # 512 kFLOP
    stale = out.read_text().replace(profsum.source_hash("fwd_step_bf16_kernel"), "0" * 16)
    out.write_text(stale)
    assert profsum.read_issued(str(out), "fwd_step_bf16_kernel") is None


def test_power_samples_parse():
    text = """GPU: 0
    POWER:
        SOCKET_POWER: 1349 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 1870 MHz
            MIN_CLK: 500 MHz
        GFX_1:
            CLK: 1792 MHz
            MIN_CLK: 500 MHz
        MEM_0:
            CLK: 2000 MHz
GPU: 0
    POWER:
        SOCKET_POWER: 1400 W
    CLOCK:
        GFX_0:
            CLK: 1641 MHz
"""
    got = profsum.parse_smi_samples(text)
    assert got == [(1349.0, [1870.0, 1792.0]), (1400.0, [1641.0])]
