"""The oracle's sizing arithmetic against the numbers the page prints."""
import json
import os

from oracle import sizing

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sizing_opt13b.json")))


def test_opt13b_bytes_per_token():
    g = GOLD["opt13b"]
    b = sizing.kv_bytes_per_token(g["layers"], g["kv_numbers_per_layer"], g["bytes_per_number"])
    assert b == g["bytes_per_token"] == 819_200
    assert b / sizing.KIB == g["kib_per_token_as_printed"]


def test_opt13b_text_and_cache():
    g = GOLD["opt13b"]
    per_tok = g["bytes_per_token"]
    text = per_tok * g["max_text_tokens"]
    assert text == 1_677_721_600
    assert round(text / sizing.GIB, 1) == g["text_cache_gb_as_printed"]
    toks = sizing.tokens_that_fit(g["cache_gb"] * sizing.GIB, per_tok)
    assert toks == 15_728
    assert abs(toks - g["tokens_in_cache_as_printed"]) / g["tokens_in_cache_as_printed"] < 0.005
    assert sizing.texts_that_fit(g["cache_gb"] * sizing.GIB, per_tok, g["max_text_tokens"]) == \
        g["texts_in_cache_as_printed"]
    assert round(g["weights_gb"] / g["card_gb"], 2) == g["weights_fraction_as_printed"]
    # decimal gigabytes would not give the printed "about 15,700"
    assert sizing.tokens_that_fit(12 * 10 ** 9, per_tok) == 14_648


def test_shared_kv_heads():
    g, o = GOLD["llama2_70b"], GOLD["opt13b"]
    b = sizing.kv_bytes_per_token_heads(g["layers_not_on_the_page"], g["kv_sets"],
                                        g["head_dim_not_on_the_page"], 2)
    assert b / sizing.KIB == g["kib_per_token_as_printed"]
    assert b / o["bytes_per_token"] == g["fraction_of_opt13b_as_printed"]
    f = GOLD["falcon_7b"]
    b = sizing.kv_bytes_per_token_heads(f["layers_not_on_the_page"], f["kv_sets"],
                                        f["head_dim_not_on_the_page"], 2)
    assert b / sizing.KIB == f["kib_per_token_as_printed"]


def test_one_layer_pool_of_the_12gb_cache():
    # 12 GiB over 40 layers, blocks of 16 tokens x 40 heads x 128 fp16, K and V
    assert sizing.blocks_per_layer(12 * sizing.GIB, 40, 40, 128, 16, 2) == 983
