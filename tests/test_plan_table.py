"""The plan table moe_default_plan uses is the tuner's measurement, not hand-copied rows
(CPU only: plan selection is host code).

- csrc/plan_table.h is exactly what `tune.py --emit` writes from the committed
  tuned_plans.json;
- for every tuned (layer, T), moe_default_plan returns the measured fastest plan, and for T
  between tuned points the plan of the nearest one (log scale, the smaller on a tie);
- a layer shape that was not tuned gets a valid plan of its weight type.
"""
import math
import os

import pytest

from moe_layer_02_amd import abi, synth, tune
from tests.test_abi_host import fake_layer

PLAN = tune.PLAN_FIELDS


@pytest.fixture(scope="module")
def data():
    return tune.load_json()


def test_header_is_generated_from_the_measurements(data):
    with open(tune.HEADER_PATH) as fh:
        assert fh.read() == tune.emit_header(data)


def test_every_layer_and_sweep_point_is_tuned(data):
    for name in ("mixtral", "qwen2", "deepseek", "scout"):
        cfg = synth.CONFIGS[name]
        L = data["layers"][name]
        assert (L["E"], L["k"], L["H"], L["I"], L["wdtype"]) == (cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype)
        assert sorted(p["T"] for p in L["points"]) == sorted(cfg.t_sweep)
        for p in L["points"]:
            assert p["best_us"] <= p["library_default_us"] + 1e-9       # the search includes the old default
            assert p["n_tried"] >= 5


def _plan(p):
    return tuple(getattr(p, f) for f in PLAN)


def _best(point):
    """A measured plan as a full tuple (plans measured before a field existed take its 0)."""
    return tuple(point["best"]) + (0,) * (len(PLAN) - len(point["best"]))


def test_default_plan_is_the_measured_best(data):
    for name, L in data["layers"].items():
        layer = fake_layer(synth.CONFIGS[name])
        pts = sorted(L["points"], key=lambda q: q["T"])
        for p in pts:
            assert _plan(abi.moe_default_plan(layer, p["T"])) == _best(p), (name, p["T"])
        for T in (3, 5, 6, 7, 12, 100, 700, 3000):          # between tuned points: the nearest
            if T > pts[-1]["T"]:
                continue
            near = min(pts, key=lambda q: (abs(math.log2(q["T"]) - math.log2(T)), q["T"]))
            assert _plan(abi.moe_default_plan(layer, T)) == _best(near), (name, T)
        big = pts[-1]["T"] * 4                                # past the largest tuned T: the largest
        assert _plan(abi.moe_default_plan(layer, big)) == _best(pts[-1])


@pytest.mark.parametrize("cfg", [synth.CONFIGS["tiny"],
                                 synth.CONFIGS["qwen2"].with_shape(E=16, k=4, H=512, I=256),
                                 synth.CONFIGS["deepseek"].with_shape(E=16, k=4, n_group=4, topk_group=2, H=768, I=512),
                                 synth.CONFIGS["mixtral"].with_shape(H=1024, I=1536)])
def test_untuned_shapes_get_valid_plans(cfg):
    layer = fake_layer(cfg)
    for T in (1, 2, 7, 64, 300, 2000):
        p = abi.moe_default_plan(layer, T)
        assert abi.moe_workspace_bytes(layer, T, p) > 0
