"""Host logic of bench.py's profiler summaries, on small synthetic counter
databases (the table rocprofv3 writes its --pmc values to): no GPU involved."""
import os
import sqlite3

import pytest

import bench


def _db(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
              "value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    c.commit()
    c.close()


def test_counter_summary_per_family(tmp_path):
    fwd, dinp = "void dtb::gemm_k64m16_kernel<0>(dtb::KParams)", "void dtb::gemm_k64_kernel<true, false, 0, true>(x)"
    attn = "void dtb::(anonymous namespace)::fwd_bf16_kernel<64, 2>(dtb::AttnP)"
    a, b = [], []
    for d, (mf, valu) in enumerate([(1000, 1600), (3000, 5000)]):  # two forward-GEMM dispatches
        a += [(fwd, d, "SQ_INSTS_MFMA", mf), (fwd, d, "SQ_INSTS_VALU", valu), (fwd, d, "SQ_INSTS_SALU", 400),
              (fwd, d, "SQ_INSTS_LDS", 200), (fwd, d, "SQ_VALU_MFMA_BUSY_CYCLES", 512.0),
              (fwd, d, "GRBM_GUI_ACTIVE", 8.0), (fwd, d, "SQ_ACTIVE_INST_VALU", 10), (fwd, d, "SQ_WAVE_CYCLES", 100)]
        b += [(fwd, d, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9), (fwd, d, "SQ_LDS_BANK_CONFLICT", 5),
              (fwd, d, "SQ_LDS_IDX_ACTIVE", 50)]
    a += [(dinp, 7, "SQ_INSTS_MFMA", 10), (dinp, 7, "SQ_INSTS_VALU", 30), (attn, 9, "SQ_INSTS_MFMA", 0),
          (attn, 9, "SQ_INSTS_VALU", 64), ("void at::native::copy_kernel", 11, "SQ_INSTS_VALU", 5)]
    _db(str(tmp_path / "a" / "p_results.db"), a)
    _db(str(tmp_path / "b" / "p_results.db"), b)
    text = bench.counter_summary(str(tmp_path), ["(commands)"])
    import json
    out = json.loads(text.split("```json\n")[1].split("\n```")[0])
    g = out["GEMM forward"]
    assert g["dispatches"] == 2
    assert g["mfma"] == pytest.approx(2000) and g["valu"] == pytest.approx(3300)
    assert g["other_valu_per_mfma"] == pytest.approx((3300 - 2000) / 2000)
    assert g["salu_per_mfma"] == pytest.approx(400 / 2000) and g["lds_per_mfma"] == pytest.approx(200 / 2000)
    assert g["mfma_busy"] == pytest.approx(512.0 / (8.0 / 8 * 1024))
    assert g["valu_active"] == pytest.approx(0.1)
    assert g["mfma_tflop"] == pytest.approx(512 * 1e9 / 1e12)
    assert g["lds_conflict"] == pytest.approx(0.1)
    # the input-gradient kernel's name is not taken for the forward kernel's, nor the reverse
    assert out["GEMM input gradient"]["mfma"] == pytest.approx(10)
    assert out["GEMM input gradient"]["other_valu_per_mfma"] == pytest.approx(2.0)
    # a family without matrix instructions has no per-MFMA ratios; foreign kernels are left out
    assert out["attention forward"]["other_valu_per_mfma"] is None
    assert "| attention forward | 1 | 0 | 64 | — |" in text
    assert len(out) == 3


def test_traffic_summary_scales_by_copy(tmp_path):
    g0, g5 = "void dtb::gemm_k64m16_kernel<0>(dtb::KParams)", "void dtb::gemm_k64m16_kernel<5>(dtb::KParams)"
    cp = "__amd_rocclr_copyBuffer"
    _db(str(tmp_path / "fetch" / "p.db"), [(g0, 1, "FETCH_SIZE", 100.0), (g5, 2, "FETCH_SIZE", 300.0),
                                           ("other", 3, "FETCH_SIZE", 1e6)])
    _db(str(tmp_path / "write" / "p.db"), [(g0, 1, "WRITE_SIZE", 50.0), (g5, 2, "WRITE_SIZE", 150.0)])
    _db(str(tmp_path / "copy_fetch" / "p.db"), [(cp, 1, "FETCH_SIZE", 512.0), (cp, 2, "FETCH_SIZE", 400.0)])
    _db(str(tmp_path / "copy_write" / "p.db"), [(cp, 1, "WRITE_SIZE", 1024.0)])
    known = 1024 * 1024
    text = bench.traffic_summary(str(tmp_path), {"workload": "w", "copy_bytes": known, "commands": ["(c)"]})
    import json
    d = json.loads(text.split("```json\n")[1].split("\n```")[0])
    assert d["dispatches"] == 2 and d["source_hash"] == bench.gemm_source_hash()
    assert d["fetch_scale"] == pytest.approx(known / (1024 * 512.0)) and d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_kib_per_dispatch"] == pytest.approx(200.0) and d["write_kib_per_dispatch"] == pytest.approx(100.0)
    assert d["traffic_bytes_per_launch"] == round((200.0 * 2.0 + 100.0 * 1.0) * 1024)
