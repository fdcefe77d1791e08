"""Pins for the oracle's closed forms against the numbers the pages print."""
import pytest

from oracle import closed_forms as cf
from oracle.block_manager import BlockManagerModel


def test_kv_bytes_llama2_7b(load_golden):
    g = load_golden("kv_cache_sizes.json")["cases"][0]
    b = cf.kv_cache_bytes(g["num_layers"], g["num_heads"], g["head_dim"],
                          g["seq_len"], g["batch"], g["dtype_bytes"])
    assert round(b / 1e9, 2) == g["printed_gb"]


def test_kv_bytes_7b_4096x16(load_golden):
    g = load_golden("kv_cache_sizes.json")["cases"][1]
    b = cf.kv_cache_bytes(g["num_layers"], g["num_heads"], g["head_dim"],
                          g["seq_len"], g["batch"], g["dtype_bytes"])
    prod = 1
    for f in g["printed_factors"]:
        prod *= f
    assert b == prod == 2 ** 35
    assert abs(b / 2 ** 30 - g["printed_approx_gb"]) < 1e-12   # 32 GiB exactly


@pytest.mark.parametrize("case", range(4))
def test_block_counts(load_golden, case):
    g = load_golden("lpnh_block_counts.json")["cases"][case]
    n, B = g["n_tokens"], g["block_size"]
    assert cf.blocks_needed(n, B) == g["blocks"]
    if "tail_tokens" in g:
        assert n - (g["blocks"] - 1) * B == g["tail_tokens"]
        assert g["full_blocks"] == g["blocks"] - 1
    if "capacity" in g:
        assert cf.blocks_needed(n, B) * B == g["capacity"]
    if "waste_fraction_printed" in g:
        # wasted slots of the tail block over the whole capacity: 10/160
        frac = cf.tail_waste_tokens(n, B) / (cf.blocks_needed(n, B) * B)
        assert frac == 10 / 160
        assert abs(100 * frac - 100 * g["waste_fraction_printed"]) <= 0.05 + 1e-12


def test_block_counts_through_the_model(load_golden):
    """The block-manager model allocates exactly the printed block counts."""
    for g in load_golden("lpnh_block_counts.json")["cases"]:
        m = BlockManagerModel(300, g["block_size"])
        m.add_sequence(0, g["n_tokens"])
        assert len(m.table(0)) == g["blocks"]
        assert m.num_free() == 300 - g["blocks"]


def test_pool_sizing(load_golden):
    g = load_golden("lpnh_pool_sizing.json")
    for gb, kb in ((1e9, 1e3), (2 ** 30, 2 ** 10), (1e9, 2 ** 10), (2 ** 30, 1e3)):
        n = cf.pool_blocks(int(g["reserved_bytes_gb"] * gb), int(g["block_bytes_kb"] * kb))
        assert abs(n - g["approx_blocks"]) / g["approx_blocks"] < 0.05


def test_block_bytes_llama_shape():
    # one block id across 32 layers at B=16 for the 7B head shape, fp16
    assert cf.block_bytes(16, 32, 32, 128, 2) == 16 * 32 * 32 * 128 * 2 * 2
    assert cf.block_bytes(16, 1, 32, 128, 2) == 256 * 1024
