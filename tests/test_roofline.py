"""The compulsory-bytes accounting reproduces the DRAM floor the KernelIndex page prints."""
import json
import os

from lm_head_linear_tiled_amd import roofline

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kernelindex_floor.json")


def test_kernelindex_dram_floor():
    g = json.load(open(GOLD))
    w = g["workload"]
    b = roofline.fwd_declared_bytes(w["N"], w["H"], w["V"], w["dtype"])
    us = roofline.floor_us(b, g["bandwidth_GBps"])
    assert round(us, 1) == g["floor_us_printed"]
    # the printed ratio uses an unrounded record time; 20.9 ms rounds it to within 0.1 %
    assert abs(g["record_ms_printed"] * 1e3 / us - g["ratio_printed"]) / g["ratio_printed"] < 1e-3


def test_flop_counts():
    assert roofline.fwd_flops(4096, 4096, 128256) == 2 * 4096 * 4096 * 128256
    assert roofline.fwdbwd_flops(1, 1, 1) == 8.0
