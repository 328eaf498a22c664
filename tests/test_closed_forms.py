"""Pins for the oracle's closed forms against the numbers the pages print.

Every fixture in tests/golden/ names the page and section it comes from.
Printed values are rounded on the pages, so each comparison states its
tolerance."""
import math
import os

import pytest

from oracle import closed_forms as cf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    """key -> list of floats, from 'key v1 v2 ...' lines ('#' starts a comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, *vals = line.split()
            out[k] = [float(v) for v in vals]
    return out


def close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


def test_tier_table():
    g = load("tier_table.txt")
    R = g["R"][0]
    for tier in ("HBM", "DRAM_PCIe4_x16", "NVMe_one_drive_share"):
        bw, ait_printed, tokens_printed = g[tier]
        assert close(cf.machine_balance(R, bw), ait_printed, 0.01), tier
        # "~32", "~2,000", "~20,900": tokens = (R/BW) / 2 since ait = 2T
        assert close(cf.tokens_needed(R, bw), tokens_printed, 0.03), tier
    # exact values behind the rounding
    assert cf.machine_balance(R, 2e12) == 62.5
    assert math.isclose(cf.tokens_needed(R, 3e9), 20833.333333, rel_tol=1e-9)


def test_ait_of_checkpointed_step():
    g = load("misc_numbers.txt")
    P, T = 7.0e9, 1234.0
    assert cf.flops_checkpointed_step(P, T) == g["step_flops_per_param_token"][0] * P * T
    assert cf.param_bytes_per_step(P) == g["param_bytes_per_param"][0] * P
    assert cf.ait_params(T) == g["ait_params_per_token"][0] * T


def test_batch_clears_nvme_bar():
    g = load("misc_numbers.txt")
    t = load("tier_table.txt")
    R, bw = t["R"][0], t["NVMe_one_drive_share"][0]
    tokens = g["batch"][0] * g["seq"][0]
    assert tokens == g["tokens"][0]
    assert cf.tier_hidden(cf.ait_params(tokens), R, bw)
    assert not cf.tier_hidden(cf.ait_params(g["seq"][0]), R, bw)
    miss = cf.machine_balance(R, bw) / cf.ait_params(g["seq"][0])
    assert close(miss, g["miss_factor_printed"][0], 0.05)


def test_adam_ait():
    g = load("misc_numbers.txt")
    assert cf.adam_ait(g["adam_flops"][0], g["adam_bytes"][0]) == g["adam_ait_printed"][0]


def test_capacity_ceiling():
    g = load("misc_numbers.txt")
    assert cf.p_max(g["node_bytes"][0]) == g["p_max_node_printed"][0]
    # "4 PB" = 64 nodes x 64 TB = 4.096e15 bytes -> 2.56e14 ("256 T")
    assert close(cf.p_max(g["nodes"][0] * g["node_bytes"][0]), g["p_max_cluster_printed"][0], 1e-9)


def test_cn_aggregate_bandwidth():
    g = load("misc_numbers.txt")
    assert g["cn_dp"][0] * g["cn_bw_one"][0] == g["cn_aggregate_printed"][0]


def test_fetch_times_and_prefetch_depth():
    g = load("fetch_and_prefetch.txt")
    layer = g["params"][0] * 2 / g["layers"][0]            # fp16 bytes per layer
    assert close(layer, g["layer_bytes_printed"][0], 0.01)  # 15.6 GB, printed 15.7
    t_own = cf.t_fetch_owner(g["layer_bytes_printed"][0], g["bw_one"][0])
    t_str = cf.t_fetch_striped(g["layer_bytes_printed"][0], int(g["dp"][0]), g["bw_one"][0])
    assert close(t_own, g["t_owner_printed"][0], 0.01)
    assert close(t_str, g["t_striped_printed"][0], 0.03)
    step = cf.flops_checkpointed_step(g["params"][0], g["tokens"][0]) / g["R"][0]
    assert close(step, g["step_s_printed"][0], 0.005)
    t_layer = step / g["layers"][0]
    assert close(t_layer, g["t_layer_printed"][0], 0.005)
    assert close(g["t_owner_printed"][0] / g["t_layer_printed"][0], g["ratio_printed"][0], 0.03)
    d = cf.prefetch_depth(g["t_owner_printed"][0], g["t_layer_printed"][0])
    assert d == g["d_owner"][0]
    assert close(cf.prefetch_buffer_bytes(d, g["layer_bytes_printed"][0]), g["buffer_bytes_printed"][0], 0.01)
    assert cf.prefetch_depth(t_str, t_layer) == g["d_striped"][0]


def test_tiling_sizes_transformer_math_page():
    g = load("tiling_sizes.txt")
    P = g["d_model"][0] * g["ffn"][0]
    assert close(P, g["params_printed"][0], 0.01)
    layer = P * 2
    assert close(layer, g["bytes_printed"][0], 0.01)
    k = int(g["k"][0])
    assert close(cf.working_bytes(layer, k), g["resident_printed"][0], 0.001)
    assert close(cf.working_bytes(layer, k, in_flight=True), g["in_flight_printed"][0], 0.01)
    # the same numbers through the tile geometry: M = 102400 split 8 ways
    n = cf.tile_cols(int(g["ffn"][0]), k)
    assert cf.tile_bytes(int(g["d_model"][0]), n) == layer / k == 655_360_000


def test_tiling_example_cn_page():
    g = load("tiling_example_cn.txt")
    hd, out, N = int(g["hd"][0]), int(g["out"][0]), int(g["N"][0])
    assert hd * out == g["params"][0]
    assert hd * out * 2 == g["weights_bytes"][0] == g["grads_bytes"][0]
    assert 2 * hd * out * 2 == g["total_bytes"][0] > g["gpu_bytes"][0]
    n = cf.tile_cols(out, N)
    assert n == g["tile_cols"][0]
    assert hd * n == g["tile_params"][0]
    assert cf.tile_bytes(hd, n) == g["tile_weight_bytes"][0]
    assert cf.weight_and_grad_tile_bytes(hd, n) == g["tile_weight_and_grad_bytes"][0]


def test_tile_geometry():
    K, M, N = 512, 2048, 4
    n = cf.tile_cols(M, N)
    assert n == 512
    assert [cf.tile_col_range(i, n) for i in range(N)] == [(0, 512), (512, 1024), (1024, 1536), (1536, 2048)]
    assert [cf.tile_host_offset(i, K, n) for i in range(N)] == [i * 524288 for i in range(N)]
    # tiles partition the host copy exactly
    assert cf.tile_host_offset(N, K, n) == K * M * 2
    with pytest.raises(ValueError):
        cf.tile_cols(100, 3)


def test_flop_counts_and_link_intensity():
    T, K, M = 4096, 8192, 32768
    assert cf.flops_fwd(T, K, M) == 2 * T * K * M
    assert cf.flops_bwd(T, K, M) == 2 * cf.flops_fwd(T, K, M)
    assert cf.link_ait_fwd(T) == T
    assert cf.link_ait_bwd(T) == 2 * T
    assert cf.link_ait_fwd_bwd(T) == 1.5 * T
    # FFN block with recompute: 8PT FLOPs over 2*(3 P1 + 2 P2) bytes = 1.6 T for P1 = P2
    P1 = P2 = 25600 * 102400
    T5 = 32768
    f = cf.flops_checkpointed_step(P1 + P2, T5)
    assert f == pytest.approx(4.194304e10 * 2 * T5 / 2 * 1.0, rel=1e-3) or f == 8 * (P1 + P2) * T5
    assert cf.ait(f, cf.ffn_tiled_h2d_bytes(P1, P2)) == pytest.approx(1.6 * T5)


def test_efficiency_model():
    assert cf.efficiency(100.0, 125e12, 32e9) == pytest.approx(100 / 3906.25)
    assert cf.efficiency(1e6, 125e12, 32e9) == 1.0
