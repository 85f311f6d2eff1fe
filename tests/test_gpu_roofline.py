"""wts_roofline(): the measured denominators are plausible and every
exchange variant selects the true maximum in every round."""
import pytest

pytestmark = pytest.mark.gpu


def test_roofline_measurements():
    from serial_draft_head_persistent_amd import roofline
    print("CASE test=roofline", flush=True)
    r = roofline(0)
    G = r["grid"]
    assert 1 <= G <= 256
    # every exchange design, every round, every workgroup: the true maximum, no expired wait
    assert r["exchange_bad"] == [0] * 6, r["exchange_bad"]
    assert all(x > 0 for x in r["exchange_us"][1:4]), r["exchange_us"]
    # rates below the chip's physical ceilings (per-CU widths at a 2.5 GHz ceiling)
    clk = r["clock_MHz"]
    assert 500 < clk < 2500, clk
    assert 0 < r["lds_read_GBps"] <= G * 256 * 2.5, r["lds_read_GBps"]            # 256 B/clk/CU
    assert 0 < r["mfma_i8_TOPs"] <= G * 4 * 2048 * 2.5e-3, r["mfma_i8_TOPs"]      # 2048 ops/clk/SIMD
    assert 0 < r["mfma_bf16_TFLOPs"] <= G * 4 * 1024 * 2.5e-3, r["mfma_bf16_TFLOPs"]
    assert 0 < r["hbm_read_GBps"] <= 8000.0, r["hbm_read_GBps"]
    assert r["hbm_read_GBps"] < r["mall_read_GBps"], (r["hbm_read_GBps"], r["mall_read_GBps"])
    # the selection round is slower than the two one-way hops it contains
    if r["exchange_us"][0] > 0 and r["hop_device_us"] > 0:
        assert r["exchange_us"][0] > r["hop_xcd_us"] + 0.5 * r["hop_device_us"]
    # a wave issues at most one VALU instruction per cycle
    assert r["valu_dep_cycles"] >= 1 and r["valu_indep_cycles"] >= 1 and r["valu_indep_4w_cycles"] >= 1
    assert r["dot4_2w_cycles"] >= 1
