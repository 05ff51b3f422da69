"""Host-side accounting of bench.py against the article's own worked example
(tests/golden/decode_bandwidth_model.json) and the closed-form work counts."""
import json
import os

import pytest

import bench
import moe_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_bandwidth_model.json")


def test_decode_bandwidth_model_matches_article():
    g = json.load(open(GOLDEN))
    est = bench.decode_tokens_per_s(g["memory_bandwidth_GB_per_s"] * 1e9, g["active_params_billion"] * 1e9,
                                    g["bytes_per_param_bf16"])
    assert round(est) == g["estimate_tokens_per_s"]                      # 800 / (3.6 * 2) = 111.1
    assert abs(est - g["measured_tokens_per_s"]) / g["measured_tokens_per_s"] < 0.05


@pytest.mark.parametrize("name,flops", [("c2", 2.886e12), ("c4", 6.228e11), ("c5", 1.305e13)])
def test_layer_flops(name, flops):
    assert abs(bench.layer_flops(W.get(name)) - flops) / flops < 2e-3


def test_layer_bytes_c5():
    wl = W.get("c5")
    assert abs(bench.layer_bytes(wl, 256) - 23.11e9) / 23.11e9 < 2e-3


def test_gateup_counts():
    wl = W.get("c2")
    assert bench.gateup_flops(wl) == 4.0 * 8192 * 4096 * 14336
    assert bench.gateup_bytes(wl, 8) == 2 * (2 * 14336 * 4096 * 8 + 8192 * 4096 + 8192 * 14336)


def test_multi_gpu_request_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_share_options_refused_before_any_gpu_work(capsys):
    """Option combinations the share measurement does not take are refused
    from the arguments alone."""
    assert bench.main(["--split-shared"]) == 2
    assert "--ep-share" in capsys.readouterr().err
    assert bench.main(["--ep-share", "8", "--workload", "c3_t8"]) == 2
    assert bench.main(["--ep-share", "3", "--workload", "c5"]) == 2        # 256 experts do not split in 3
    assert bench.main(["--workload", "c3mx_t8", "--mode", "grouped"]) == 2
    assert bench.main(["--ep-index", "1"]) == 2
    assert bench.main(["--ep-share", "4", "--ep-index", "4", "--workload", "c5"]) == 2
    assert bench.main(["--ep-balanced"]) == 2
    assert bench.main(["--ep-share", "8", "--ep-balanced", "--ep-interleave"]) == 2


def test_layer_flops_shared_slice():
    """A share that runs the shared expert on T/N tokens counts its FLOPs
    for those tokens only."""
    wl = W.get("c5")
    full = bench.layer_flops(wl)
    part = bench.layer_flops(wl, Ts=wl.T // 8)
    assert full - part == 6.0 * (wl.T - wl.T // 8) * wl.d * wl.f_shared


def test_tile_work():
    wl = W.get("c2")
    # 1000 rows -> 1024 at 32-row fragments and at 256-row tiles; 40 -> 64 and 256; 0 rows: no tiles
    tw = bench.tile_work(wl, [1000, 40, 0])
    assert tw["gateup"] == tw["down"] == 1088 / 1040            # f and d fill whole output tiles
    assert tw["rows_at_256_row_tiles"] == 1280 / 1040
    assert bench.tile_work(wl, [256, 512])["gateup"] == 1.0
    assert bench.tile_work(wl, [0, 0])["down"] is None
