"""The oracle's memory and communication accounting against the numbers the
pages print (tests/golden/accounting.json, each entry with its citation)."""
import json
import os

import pytest

import oracle

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "accounting.json")))


def test_sixteen_bytes_per_parameter():
    b = G["bytes_per_param"]
    assert b["weight"] + b["grad"] + b["optimizer"] == b["total"] == 16
    for n in (1.0, 7e9, 123456.0):
        assert oracle.model_state_bytes(n, 1, 0, b["optimizer"]) == b["total"] * n
        # stage 3 on n_dp ranks: 16 N / n_dp per rank
        assert oracle.model_state_bytes(n, 8, 3, 12) == pytest.approx(16 * n / 8, rel=1e-15)


@pytest.mark.parametrize("e", G["state_memory"], ids=lambda e: f"{e['n']:.3g}-{e['n_dp']}-s{e['stage']}")
def test_printed_state_memory(e):
    got = oracle.model_state_bytes(e["n"], e["n_dp"], e["stage"], 12) / 1e9
    assert abs(got - e["gb"]) <= e["abs_tol_gb"], e["cite"]


@pytest.mark.parametrize("e", G["weights_only"])
def test_printed_weight_memory(e):
    assert abs(e["n"] * e["bytes_per"] / 1e9 - e["gb"]) <= e["abs_tol_gb"]


@pytest.mark.parametrize("e", G["headroom"])
def test_printed_headroom(e):
    used = oracle.model_state_bytes(e["n"], e["n_dp"], e["stage"], 12) / 1e9
    assert abs((e["capacity_gb"] - used) - e["left_gb"]) <= e["abs_tol_gb"]


def test_asymptotes_and_stage1_saving():
    lim = G["asymptotes"]["bytes_per_param_limit"]
    for stage in range(4):
        per = oracle.model_state_bytes(1.0, 1e12, stage, 12)
        assert per == pytest.approx(lim[stage], abs=1e-9)
    k = G["stage1_saving"]["k"]
    for n_dp in (2, 8, 64):
        saved = oracle.model_state_bytes(1e9, n_dp, 0, k) - oracle.model_state_bytes(1e9, n_dp, 1, k)
        assert saved == pytest.approx(k * 1e9 * (1 - 1 / n_dp), rel=1e-15)


@pytest.mark.parametrize("e", G["comm"])
def test_printed_comm_bytes(e):
    got = oracle.comm_bytes(e["n"], e["n_dp"], e["stage"], e["param_bytes"], e["grad_bytes"]) / 1e9
    assert abs(got - e["gb"]) <= e["abs_tol_gb"], e["cite"]


def test_comm_ratios():
    lim = G["comm_ratios"]["stage_over_dp_limit"]
    dp = oracle.comm_bytes(1e9, 1e9, 0)
    for stage in range(4):
        assert oracle.comm_bytes(1e9, 1e9, stage) / dp == pytest.approx(lim[stage], rel=1e-8)
    # n_dp = 1 sends nothing; mixed element sizes enter per collective
    assert oracle.comm_bytes(1e9, 1, 2) == 0
    assert oracle.comm_bytes(8, 8, 1, param_bytes=2, grad_bytes=4) == 7 * 4 + 7 * 2


def test_invalid_stage():
    assert oracle.model_state_bytes(1e9, 8, 4, 12) == -1
    assert oracle.comm_bytes(1e9, 8, -1) == -1
