"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the traffic records'
source check, the flop count of tree attention and the matrix-core counter summary."""
import json
import os
import types

import numpy as np
import pytest

import bench
import oracle


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_record_needs_the_current_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    hdr = tmp_path / "common.h"
    src.write_text("// kernel v1\n")
    hdr.write_text("// header\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "COMMON_HEADER", "common.h")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"k": "kernel.hip"})
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench._traffic("k") is None                       # no record
    rec = {"bytes_per_launch": 123, "source_sha256_16": bench._src_hash("kernel.hip")}
    (tmp_path / "k_C5_traffic.json").write_text(json.dumps(rec))
    assert bench._traffic("k") == 123
    src.write_text("// kernel v2\n")                        # the kernel changed since
    assert bench._traffic("k") is None
    src.write_text("// kernel v1\n")
    hdr.write_text("// header changed\n")                   # so did the header it includes
    assert bench._traffic("k") is None


@pytest.mark.parametrize("seed", range(3))
def test_attention_flops_count_every_visible_key(seed):
    """4*D flops per (query row, visible key); node i sees the prefix and its root path
    (the oracle's ancestor-or-self sets), for every query head."""
    rng = np.random.default_rng(seed)
    B, N, P, D, Hq = 3, 17, 50, 64, 6
    parents = np.stack([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)])
    cfg = types.SimpleNamespace(N=N, P=P, D=D, Hq=Hq)
    keys = sum(P + len(oracle.ancestor_sets(list(parents[b]))[i]) for b in range(B) for i in range(N))
    assert bench.attn_flops(parents, cfg) == 4.0 * D * Hq * keys


def test_mfma_summary_from_counters(tmp_path, monkeypatch):
    """Two dispatches of one kernel: clock = GUI-active cycles per XCC over the dispatch
    time, MFMA busy = busy cycles per SIMD over those cycles, rate = MOPS * 512 / time."""
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    name = "void eagle::(anonymous namespace)::lm_head_gemm<4, 2, 4, 2, 3>(unsigned short const*)"
    rows = []
    for disp, (t0, dur_ns) in enumerate([(1_000, 500_000), (2_000_000, 400_000)]):
        cycles = 2.0e9 * dur_ns * 1e-9          # a 2 GHz clock
        vals = {"GRBM_GUI_ACTIVE": 8 * cycles, "GRBM_COUNT": 8 * cycles,
                "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * 1024,
                "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.0e12 * dur_ns * 1e-9 / 512,
                "SQ_BUSY_CU_CYCLES": 0.0, "SQ_LDS_IDX_ACTIVE": 0.25 * cycles * 256,
                "SQ_LDS_BANK_CONFLICT": 0.0, "SQ_INSTS_LDS": 0.0}
        for k, v in vals.items():
            rows.append(f'{disp},"{name}","{k}",{v},{t0},{t0 + dur_ns}')
    path = tmp_path / "counters.csv"
    path.write_text('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value","Start_Timestamp",'
                    '"End_Timestamp"\n' + "\n".join(rows) + "\n")
    text = bench.summarize_mfma(str(path))
    line = [l for l in text.splitlines() if l.startswith("| lm_head_gemm")][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "2"                        # dispatches
    assert cells[2] == "450.0"                    # mean duration, us
    assert cells[3] == "2000"                     # clock, MHz
    assert cells[4] == "50.0"                     # MFMA busy %
    assert cells[5] == "1"                        # bf16 TFLOP/s (1e12 flop/s)
    assert cells[6] == str(round(1024 * 1024 * 2.0e9 / 1e12))   # peak at that clock
    assert cells[7] == "25.0"                     # LDS active %
    assert os.path.exists(tmp_path / bench.MFMA_MD)


def test_host_info_names_the_cpu():
    info = bench._host_info()
    assert set(info) == {"cpu_model", "usable_cores", "machine_cores"}
    assert 1 <= info["usable_cores"] <= info["machine_cores"]
    assert isinstance(info["cpu_model"], str) and info["cpu_model"]


def test_trace_summary_keeps_the_timed_steps(tmp_path):
    """A per-step kernel's warmup dispatches (slow here) are left out of the trace
    summary; a kernel with another dispatch count keeps all of its dispatches."""
    path = tmp_path / "run_kernel_trace.csv"
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for i in range(8):   # 2 warmup steps, 3 timed as a whole, 3 timed call by call
        dur = 900_000 if i < 2 else 500_000
        rows.append(f"step_kernel,{t},{t + dur}")
        t += dur + 1000
        if i == 0:
            rows.append(f"once_kernel,{t},{t + 7000}")
            t += 8000
    path.write_text("\n".join(rows) + "\n")
    stats = {st[0]: st for st in bench.step_kernel_stats(str(path), 2, 3)}
    assert stats["step_kernel"][1:5] == (6, 500.0, 500.0, 500.0)
    assert stats["once_kernel"][1:3] == (1, 7.0)
