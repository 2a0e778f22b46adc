"""The pages' printed parameter counts and prefix-scratch sizes, reproduced
from the parameter set and the summary layout (12 bytes per real channel per
chunk summary or group summary)."""
import json
import math
import os

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_tables.json")))


def samu_parameter_count(D):
    # w_phi, w_r over the D+1 entries of [x_sel; 1]; a_phi, a_r; nu, theta per mode
    M = D // 2
    return 2 * (D + 1) + 2 + 2 * M


def rglru_parameter_count(D, blocks):
    # two block-diagonal gate layers (blocks x (D/blocks)^2 weights + D biases) and alpha
    return 2 * (blocks * (D // blocks) ** 2 + D) + D


def test_parameter_counts():
    for row in GOLD["mixer_parameters"]:
        assert samu_parameter_count(row["D"]) == row["samu"]
        assert rglru_parameter_count(row["D"], GOLD["rglru_gate_blocks"]) == row["rglru"]


def scratch_mib(B, L, D, K, G, serial):
    C = math.ceil(L / K)
    groups = 0 if serial else math.ceil(C / G)
    return GOLD["prefix_scratch_formula"]["bytes_per_real_channel_per_summary"] * B * D * (C + groups) / 2**20


def test_prefix_scratch_table():
    f = GOLD["prefix_scratch_formula"]
    for row in GOLD["prefix_scratch_mib"]:
        s = scratch_mib(row["B"], row["L"], row["D"], f["samu_chunk"], f["samu_group_chunks"],
                        row["samu_serial"])
        r = scratch_mib(row["B"], row["L"], row["D"], f["rglru_chunk"], f["rglru_group_chunks"], False)
        assert round(s, f["mib_decimals"]) == row["samu"]
        assert round(r, f["mib_decimals"]) == row["rglru"]
