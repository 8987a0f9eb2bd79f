"""Memory-capacity model (bit_rotated_kv_split_amd/capacity.py)."""
import math

import pytest

from bit_rotated_kv_split_amd import capacity as cap


def test_bits_per_element_matches_the_printed_figures():
    # 2.28 bits at 128K (page "Together AI 开源 OSCAR…", section "结果") and
    # 2.38 BPE at 32K (page "超越TurboQuant…", the Qwen3-8B comparison), G = 128
    assert round(cap.bits_per_element(131072, 128), 2) == 2.28
    assert round(cap.bits_per_element(32768, 128), 2) == 2.38


@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("context", [320 + 64, 320 + 64 * 1000, 131072])
def test_request_bytes_agree_with_bits_per_element(group, context):
    s = cap.QWEN3_8B
    elems = s.layers * s.kv_heads * 2 * 128 * context
    assert (context - 320) % 64 == 0
    assert cap.request_kv_bytes(s, context, "int2", group) * 8 == pytest.approx(
        cap.bits_per_element(context, group) * elems, rel=1e-12)
    assert cap.request_kv_bytes(s, context, "bf16", group) == s.layers * s.kv_heads * 512 * 64 * math.ceil(
        context / 64)


def test_qwen3_8b_weights():
    s = cap.QWEN3_8B
    assert 8.15e9 < s.weight_bytes() / 2 < 8.25e9            # published size: 8.2B parameters
    assert s.weight_bytes() - s.weight_bytes_per_step() == 2 * s.vocab * s.hidden


def test_concurrency_and_waves():
    s = cap.QWEN3_8B
    per = cap.request_kv_bytes(s, 100_000, "bf16")
    budget = s.weight_bytes() + 1e9 + 17 * per + per / 2
    assert cap.concurrency(s, budget, 1e9, 100_000, "bf16") == 17
    assert cap.concurrency(s, s.weight_bytes(), 1e9, 100_000, "bf16") == 0
    assert cap.wave_batches(32, 17) == [17, 15]
    assert cap.wave_batches(32, 40) == [32]
    assert cap.wave_batches(6, 3) == [3, 3]
    assert cap.wave_batches(5, 0) == []


def test_model_rows_with_linear_attention_time():
    s = cap.QWEN3_8B
    seen = []

    def attn(mode, b):
        seen.append((mode, b))
        return (100.0 if mode == "int2" else 700.0) * b

    rows = cap.model_rows(s, 100_000, 32, [288], 8.0, 128, attn, 5000.0)
    r = rows[0]
    assert r["int2"]["waves"] == [32] and r["bf16"]["waves"] == [17, 15]
    dense = s.weight_bytes_per_step() / 5e12
    int2_s = s.layers * 100e-6 * 32 + dense
    bf16_s = sum(s.layers * 700e-6 * b + dense for b in (17, 15))
    assert r["job_throughput_ratio"] == round(round(32 / int2_s, 1) / round(32 / bf16_s, 1), 2)
    assert ("bf16", 17) in seen and ("bf16", 15) in seen and ("int2", 32) in seen
