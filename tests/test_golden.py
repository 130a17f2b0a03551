"""Figures printed on the pages, used as fixed values (no GPU)."""
import json
import os

from linear_cross_entropy_07_amd import inputs

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def test_llmc_softmax_tensor_size_matches_gpt2_workload():
    f = G["llmc_softmax_tensor"]
    nbytes = f["batch"] * f["seq"] * f["vocab"] * f["item_bytes"]
    assert abs(nbytes - f["approx_bytes_stated"]) / f["approx_bytes_stated"] < 0.1
    w = inputs.WORKLOADS["gpt2_head"]
    assert (w.BT, w.H, w.V) == (f["batch"] * f["seq"], f["channels"], f["vocab"])


def test_ragged_protocol_bounds():
    f = G["ragged_bt_protocol"]
    bts = inputs.ragged_bt_list(seed=0, draws=20)
    assert bts[0] == f["first"] and bts[-1] == f["last"] and len(bts) == 22
    for bt in bts[1:-1]:
        assert f["low"] <= bt <= f["high_inclusive"] + f["jitter_inclusive"]
    w = inputs.WORKLOADS["ragged"]
    assert (w.H, w.V) == (f["H"], f["V"])
    # the page's point: B*T is generally not a multiple of the chunk size
    assert any(bt % f["chunk_size"] for bt in bts)
