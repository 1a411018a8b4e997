"""The work/traffic closed forms reproduce every number the pages print (no GPU)."""
import json
import os

import pytest

from tiled_online_softmax_causal_amd import costmodel as cm


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_logical_traffic_sweep(golden_dir):
    """aiml.sh run-output.txt hbm_traffic_sweep: all 4 rows, all MB figures, q-block counts."""
    for row in _golden(golden_dir, "page_traffic_sweep.json")["rows"]:
        t = cm.page_logical_traffic(row["seq_len"], row["num_heads"], row["head_dim"], 2, 128)
        assert round(t["qkvo_bytes"] / 1e6, 2) == row["standard_qkv_o_mb"]
        assert round(t["qkvo_bytes"] / 1e6, 2) == row["qkvo_compulsory_bytes_mb"]
        assert round(t["nxn_bytes"] / 1e6, 2) == row["standard_nxn_matrix_hbm_mb"]
        assert round(t["standard_total_bytes"] / 1e6, 2) == row["standard_total_hbm_mb"]
        assert round(t["tiled_logical_bytes"] / 1e6, 2) == row["tiled_logical_access_mb_no_cache_reuse"]
        assert t["num_q_blocks"] == row["num_q_blocks"]


def test_reduced_order_roofline(golden_dir):
    """chipfoundryservices.com 'FlashAttention' model outputs at b8 h32 S8192 d128."""
    g = _golden(golden_dir, "page_roofline_model.json")
    i, o = g["inputs"], g["outputs"]
    r = cm.page_roofline(i["batch_size"], i["num_heads"], i["seq_length"], i["head_dim"],
                         i["elem_bytes"], i["compute_tops"] * 1e12, i["hbm_bandwidth_gb_s"] * 1e9,
                         causal=bool(i["causal"]), sram_bytes=i["sram_kb"] * 1024, block=i["block_size"])
    assert round(r["flops"] / 1e9, 2) == o["flops_gflop"]
    assert round(r["scores_bytes"] / 1e9, 4) == o["scores_matrix_gb"]
    assert round(r["naive_bytes"] / 1e9, 4) == o["naive_hbm_gb"]
    assert round(r["fa_bytes"] / 1e9, 4) == o["fa_hbm_gb"]
    assert round(r["hbm_reduction"], 1) == o["hbm_reduction_x"]
    assert round(r["machine_balance"], 1) == o["machine_balance_flop_byte"]
    assert round(r["ai_fa"], 1) == o["arithmetic_intensity_fa"]
    assert round(r["ai_naive"], 1) == o["arithmetic_intensity_naive"]
    assert r["fa_bound"] == o["fa_bottleneck"] and r["naive_bound"] == o["naive_bottleneck"]
    assert round(r["naive_time_s"] * 1e3, 3) == o["naive_time_ms"]
    assert round(r["fa_time_s"] * 1e3, 3) == o["fa_time_ms"]
    assert round(r["speedup"], 2) == o["speedup_x"]
    assert round(r["fa_flops_per_s"] / 1e12, 1) == o["fa_tflops"]
    assert r["sram_needed_bytes"] / 1024 == o["sram_needed_kb"]
    assert r["max_block_sram"] == o["max_block_sram"]
    assert r["sram_fit"] == o["sram_fit"]
    assert r["q_blocks"] == o["q_blocks"]


def test_reduced_order_profile_curves(golden_dir):
    g = _golden(golden_dir, "page_roofline_model.json")
    i, pp = g["inputs"], g["profile_points"]
    seqs = cm.page_profile_seqs(pp["first_seq"], pp["last_seq"], pp["n_points"])
    grid = {round(s, 1): s for s in seqs}
    for key, field in (("reduction_vs_seq", "hbm_reduction"), ("speedup_vs_seq", "speedup")):
        for s_printed, val in pp[key]:
            s = grid[s_printed]
            r = cm.page_roofline(i["batch_size"], i["num_heads"], s, i["head_dim"], i["elem_bytes"],
                                 i["compute_tops"] * 1e12, i["hbm_bandwidth_gb_s"] * 1e9)
            assert round(r[field], 3) == pytest.approx(val, abs=1e-9)


def test_flop_and_byte_conventions():
    # the headline workload: b8 h32 S8192 d128 bf16 causal
    assert cm.attention_flops(8, 32, 8192, 128, True) == pytest.approx(4398.046511104e9)
    assert cm.attention_flops(1, 32, 4096, 128, False) == 2 * cm.attention_flops(1, 32, 4096, 128, True)
    assert cm.algorithmic_bytes(8, 32, 8192, 128, 2, with_lse=False) == 2147483648
    assert cm.algorithmic_bytes(8, 32, 8192, 128, 2) == 2147483648 + 4 * 8 * 32 * 8192


def test_tile_counts():
    # the page's example visits 10 tiles at S=64 with 16x16 blocks
    assert cm.causal_kv_tiles(64, 16, 16) == 10
    assert cm.causal_kv_tiles(64, 16, 16, causal=False) == 16
    # S=8192, 128-row query blocks, 64-key tiles: 2(qb+1) tiles for each of 64 blocks
    assert cm.causal_kv_tiles(8192, 128, 64) == sum(2 * (qb + 1) for qb in range(64))
    assert cm.causal_kv_tiles(65, 16, 16) == 15
