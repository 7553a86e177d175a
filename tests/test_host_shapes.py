"""Host logic: GEMM shapes derived from the model configuration, checked against
the values printed on the page (tests/golden/codonfm5b_config.json)."""

import json
import os

from fp8_precision_transformer_amd.shapes import CODONFM_5B, ModelConfig, layer_flops, layer_gemms

GOLD = os.path.join(os.path.dirname(__file__), "golden", "codonfm5b_config.json")


def test_codonfm5b_shapes_match_page():
    with open(GOLD) as f:
        g = json.load(f)
    cfg = ModelConfig(g["hidden_size"], g["intermediate_size"], g["num_attention_heads"],
                      g["num_hidden_layers"], g["micro_batch_size"], g["sequence_length"])
    assert cfg == CODONFM_5B
    assert cfg.tokens == g["tokens_M"]
    gemms = layer_gemms(cfg)
    assert len(gemms) == g["gemm_shapes_per_layer"]
    by = {(x.weight, x.stage): x for x in gemms}
    qf, qd = by[("qkv", "fprop")], by[("qkv", "dgrad")]
    assert (qf.k, qf.n) == (g["qkv_fprop_K"], g["qkv_fprop_N"])
    # Dgrad swaps K and N
    assert (qd.k, qd.n) == (g["qkv_fprop_N"], g["qkv_fprop_K"])
    ao = by[("attn_out", "fprop")]
    assert [ao.n, ao.k] == g["attn_out_weight"]
    # Wgrad reduces over the tokens
    assert all(x.k == cfg.tokens for x in gemms if x.stage == "wgrad")
    # every GEMM of a layer has the same flop count per weight across the 3 stages
    for w in ("qkv", "attn_out", "mlp_up", "mlp_down"):
        assert len({by[(w, s)].flops for s in ("fprop", "dgrad", "wgrad")}) == 1
    assert layer_flops(cfg) == 3 * 2 * cfg.tokens * (4096 * 12288 + 4096 * 4096 + 2 * 4096 * 16384)
