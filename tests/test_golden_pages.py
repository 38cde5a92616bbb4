"""The oracle's byte model against figures printed on the pages (CPU)."""

import json
import os

from oracle import quant
from paged_kv_attention_walk_amd import synth


def _load(golden_dir, name):
    return json.load(open(os.path.join(golden_dir, name)))


def test_capacity_figures(golden_dir):
    fx = _load(golden_dir, "capacity_lucebox555.json")
    per_slot = fx["n_kv_heads"] * 2 * quant.row_bytes(fx["kind"], fx["head_dim"])
    mib, gib = 2.0 ** 20, 2.0 ** 30
    tol = fx["printed_precision"]
    assert sum(synth.RAGGED_LENS) == fx["live_tokens"]
    assert 8 * max(synth.RAGGED_LENS) == fx["padded_slots"]
    assert abs(fx["padded_slots"] * per_slot / mib - fx["one_layer_mib"]["padded"]) <= tol["one_layer_mib"]
    assert abs(fx["live_tokens"] * per_slot / mib - fx["one_layer_mib"]["paged"]) <= tol["one_layer_mib"]
    assert abs(16 * fx["padded_slots"] * per_slot / gib - fx["sixteen_layers_gib"]["padded"]) <= tol["sixteen_layers_gib"]
    assert abs(16 * fx["live_tokens"] * per_slot / gib - fx["sixteen_layers_gib"]["paged"]) <= tol["sixteen_layers_gib"]
    assert abs(fx["padded_slots"] / fx["live_tokens"] - fx["less_kv_factor"]) <= tol["less_kv_factor"]
    assert abs(100 * (1 - fx["live_tokens"] / fx["padded_slots"]) - fx["saving_percent"]) <= tol["saving_percent"]


def test_rdna4_bandwidth_figures(golden_dir):
    fx = _load(golden_dir, "rdna4_decode_timings_llamacpp_pr2.json")
    per_tok = fx["n_kv_heads"] * (quant.row_bytes(fx["k_kind"]) + quant.row_bytes(fx["v_kind"]))
    assert per_tok == 1664
    # the stated bandwidths describe the kernel before the commit's change
    for label, us in fx["us_per_call"]["before"].items():
        ctx = fx["context_labels"][label]
        gbps = [ctx * per_tok / (u * 1e-6) / 1e9 for u in us]
        assert 570 <= gbps[0] <= 610, (label, gbps)
        assert all(370 <= g <= 410 for g in gbps[1:]), (label, gbps)
    # a wrong row size would leave the band: 256-byte Q8_0 rows (no scales)
    # or 4-byte scales
    for bad in (4 * (256 + 144), 4 * (288 + 144)):
        ok = all(570 <= fx["context_labels"][lb] * bad / (us[0] * 1e-6) / 1e9 <= 610
                 for lb, us in fx["us_per_call"]["before"].items())
        assert not ok
