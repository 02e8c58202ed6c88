"""Host-side checks of bench.py's per-block timing summary (no GPU)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _records(blocks, cus, kt, pro, loop, epi, gap, ghz, grid=None, stale=0):
    """Synthetic records: `blocks` blocks over `cus` CUs, each CU running its
    blocks back to back; times in microseconds, clock in GHz."""
    rec = np.zeros((blocks + stale, 8), dtype=np.uint64)
    per = blocks // cus
    for b in range(blocks):
        cu, i = b % cus, b // cus
        t0 = 1_000_000 + i * (pro + loop + epi + gap) * 100
        t1 = t0 + pro * 100
        t2 = t1 + loop * 100
        t3 = t2 + epi * 100
        c0 = 5_000_000
        c3 = c0 + (t3 - t0) / 100 * ghz * 1e3
        rec[b] = [int(t0), int(t1), int(t2), int(t3), int(c0), int(c3), (cu << 8) | (1 << 32),
                  (grid or blocks) | (kt << 32)]
    for b in range(blocks, blocks + stale):  # slots of an older, larger launch
        rec[b] = [10, 20, 30, 40, 1, 2, 0, (blocks + stale) | (kt << 32)]
    assert per * cus == blocks
    return rec


def test_block_timing_report_recovers_the_phases():
    rec = _records(blocks=64, cus=16, kt=65, pro=3.0, loop=100.0, epi=7.5, gap=0.5, ghz=1.5)
    r = bench.block_timing_report(rec, "gemm_nn_act_fwd")
    assert r["blocks"] == 64 and r["cus"] == 16 and r["tiles_per_cu"] == 4
    assert abs(r["prologue_us"] - 3.0) < 0.02 and abs(r["k_loop_us"] - 100.0) < 0.02
    assert abs(r["epilogue_us"] - 7.5) < 0.02 and abs(r["gap_between_blocks_us"] - 0.5) < 0.02
    assert abs(r["clock_GHz"] - 1.5) < 1e-3
    # 100 us x 1.5 GHz / 65 steps
    assert abs(r["cycles_per_k_step"] - 100.0 * 1500 / 65) < 1.0
    assert abs(r["k_loop_mfma_issue_frac"] - 2048 / (100.0 * 1500 / 65)) < 1e-3


def test_block_timing_report_ignores_slots_of_older_launches():
    rec = _records(blocks=32, cus=8, kt=10, pro=2.0, loop=20.0, epi=1.0, gap=0.0, ghz=2.0, stale=16)
    r = bench.block_timing_report(rec, "gemm_nn_store")
    assert r["blocks"] == 32 and r["grid"] == 32


def test_block_timing_report_empty_slot():
    assert bench.block_timing_report(np.zeros((16, 8), dtype=np.uint64), "x") is None


def test_timing_family_names():
    from workload import CONFIGS
    assert bench.timing_family_names(CONFIGS[2])[:4] == ["gemm_nn_act_fwd", "gemm_nt_act_bwd", "gemm_nt_store",
                                                         "gemm_nn_store"]
    assert bench.timing_family_names(CONFIGS[6])[0] == "gemm_nn_relu2_fwd"
    assert bench.timing_family_names(CONFIGS[4])[4] == "gemm_nn_act_fwd_nf4"


def test_only_the_timing_build_exports_block_times():
    import ctypes

    import pytest

    pkg = os.path.join(ROOT, "adapter_mlp_amd")
    normal, timing = (os.path.join(pkg, n) for n in ("liblora_mi355x.so", "liblora_mi355x_timing.so"))
    if not (os.path.exists(normal) and os.path.exists(timing)):
        pytest.skip("libraries not built")
    assert hasattr(ctypes.CDLL(timing), "lora_block_times")
    assert not hasattr(ctypes.CDLL(normal), "lora_block_times")


def test_phase_timing_report():
    rec = np.zeros((64, 2, 8), dtype=np.uint64)
    for b in range(64):
        base = 10_000 + 50 * b
        # group 0: MFMA 1100, wait 10, barrier 80, read 900, barrier 200 (step 2290)
        rec[b, 0, :7] = [base, base + 1100, base + 1110, base + 1190, base + 2090, base + 2290, 65]
        # group 1: read 1000, barrier 190, MFMA 1000, then the next step at +2290
        rec[b, 1, :7] = [base + 1190 - 2290 + 2290, base + 2190, base + 2380, base + 3380, 0, base + 3480, 65]
    r = bench.phase_timing_report(rec, "gemm_nn_store")
    assert r["blocks"] == 64 and r["k_steps"] == 65
    assert r["cycles_per_k_step"] == 2290.0
    assert (r["g0_mfma"], r["g0_load_wait"], r["g0_barrier_after_mfma"], r["g0_read"], r["g0_barrier_after_read"]) == \
        (1100.0, 10.0, 80.0, 900.0, 200.0)
    assert (r["g1_read"], r["g1_barrier_after_read"], r["g1_mfma"], r["g1_barrier_after_mfma"]) == (1000.0, 190.0, 1000.0, 100.0)
    assert bench.phase_timing_report(np.zeros((64, 2, 8), dtype=np.uint64), "x") is None
