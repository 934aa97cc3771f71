"""Size accounting pinned to the memory arithmetic the pages print
(tests/golden/page_memory_arithmetic.txt), evaluated with the oracle's format table."""
import os

import oracle as O

GiB = 2.0 ** 30
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_memory_arithmetic.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, val = line.split()[:2]
        out[name] = float(val)
    return out


def row_bytes(fmt):
    N, kind, cb, sb, pb = O.format_info(fmt)
    return cb + sb + pb // 128


def test_first_page_arithmetic():
    g = golden()
    per_tok = 2 * 64 * 8 * row_bytes(O.BF16)               # K and V, 64 layers, 8 heads
    assert per_tok == g["fp16_bytes_per_token_64l_8h_128d"]
    assert round(per_tok * 240000 / GiB) == 59 and int(per_tok * 240000 / GiB) == g["fp16_cache_240000_tokens_gib"]
    data4 = 2 * 64 * 8 * O.format_info(O.Q4_0)[2]          # 4-bit codes only
    assert data4 == g["q4_bytes_per_token_no_overhead_kib"] * 1024
    assert round(data4 * 240000 / GiB) == g["q4_cache_240000_tokens_gib"]
    # a tail of T FP16 tokens adds T * (per_tok - data4) on top of the 4-bit cache
    add1k = 1024 * (per_tok - data4) / GiB
    add20k = 20000 * (per_tok - data4) / GiB
    assert abs((15 + add1k) - g["q4_plus_fp16_tail_1k_gib"]) < 0.05
    assert abs((15 + add20k) - g["q4_plus_fp16_tail_20k_gib"]) < 0.05
    assert round(100 * 1024 / 240000, 1) == g["tail_1k_fraction_of_240k_percent"]


def test_second_page_arithmetic():
    g = golden()
    per_tok = 2 * 32 * 32 * row_bytes(O.BF16)              # hidden 4096 = 32 heads x 128, 32 layers
    assert per_tok == g["bf16_bytes_per_token_hidden4096_32l_kib"] * 1024
    assert per_tok * 1024 == g["bf16_tail_1024_mib"] * 2**20
    assert per_tok * 32768 == g["bf16_cache_32k_gib"] * GiB
    # q6 against q8 "saves 20-25%"
    for f6, f8 in ((O.Q6_0, O.Q8_0), (O.Q6_1, O.Q8_1)):
        saving = 100 * (1 - row_bytes(f6) / row_bytes(f8))
        assert g["q6_vs_q8_saving_percent_lo"] <= saving <= g["q6_vs_q8_saving_percent_hi"]
