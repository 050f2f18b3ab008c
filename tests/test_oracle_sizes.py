"""Pins of the closed-form shard sizes against the sizes the pages print."""
import json
import os

from oracle import sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "store_sizes.json")))
UNIT = {"GB": 1e9, "MB": 1e6, "GiB": 2 ** 30}


def _round(x, digits):
    return round(x, digits)


def test_store_sizes_reproduce_the_printed_figures():
    for e in GOLD["entries"]:
        total = e["layers"] * sizes.layer_bytes_pages(tuple(e["shape"]), e["quant"])
        assert _round(total / UNIT[e["unit"]], e["digits"]) == e["value"], e["what"]


def test_embed_head_and_grown_store():
    eh = GOLD["embed_head"]
    both = 2 * sizes.embed_bytes(eh["vocab"], eh["hidden"])
    assert _round(both / 1e9, 2) == eh["value"]
    store8 = 32 * sizes.layer_bytes_pages((4096, 32, 8, 128, 14336, False), "nf4")
    assert _round((store8 + both) / 1e9, 2) == GOLD["store_with_embed_head"]["value"]


def test_fp32_absmax_layout_is_the_documented_ratio():
    shape = (4096, 32, 8, 128, 14336, False)
    lin = sizes.layer_linear_params(*shape[:5])
    assert lin == 218103808
    assert sizes.layer_bytes_fp32_absmax(shape) == lin * 9 // 16 + 4 * 4096
