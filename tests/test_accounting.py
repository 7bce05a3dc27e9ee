"""Host-side byte accounting, pinned to the pages' bandwidth arithmetic.

Pins (derived from printed numbers, each cited):
 * Uzu page (fange-kb.cn), "Why batch-one decoding is memory-bound":
   153 GB/s over a 5.2 GB checkpoint gives about 29 tok/s.
 * "MLX Runner: An Inference Engine You Can Read", "Optimized against a known
   ceiling": 197 GB/s over 4.08 GB gives about 48 tok/s; 41.0 tok/s is about
   85% of it.
 * Same page, "Architecture: one command buffer per token": storing the scales
   and biases a second time adds about a ninth -- for 4-bit group-64 with fp16
   scale + bias that is 0.5 of 4.5 bits per weight.
 * Deltafin page (aihot.virxact.com), install section and I/O list: 16 experts
   x 92 layers = 25.8 GB per token, one expert = one 17.55 MB range.  With
   MXFP4 at 4.25 bits per weight and an expert of three 7168 x 1536 matrices
   that is 17,547,264 bytes per expert (the 7168 x 1536 shape is a reading:
   only the byte totals are printed).
"""
import pytest

from quantized_weight_decode_dequant_amd import roofline as R
from quantized_weight_decode_dequant_amd import synth


def test_uzu_ceiling():
    assert R.decode_tok_per_s(153, 5.2e9) == pytest.approx(29.4, abs=0.05)


def test_mlx_runner_ceiling_and_fraction():
    bound = R.decode_tok_per_s(197, 4.08e9)
    assert bound == pytest.approx(48.3, abs=0.05)
    assert 41.0 / bound == pytest.approx(0.849, abs=0.001)


def test_q4_scale_bias_overhead_is_a_ninth():
    bits = R.Q4_BYTES_PER_WEIGHT * 8
    assert bits == 4.5
    assert (bits - 4.0) / bits == pytest.approx(1 / 9)


def test_deltafin_expert_bytes():
    per_expert = R.moe_expert_bytes(7168, 1536)
    assert per_expert == 17547264
    assert per_expert / 1e6 == pytest.approx(17.55, abs=0.01)
    assert 16 * 92 * per_expert / 1e9 == pytest.approx(25.8, abs=0.05)


def test_decode_step_bytes():
    shapes = synth.decode_step_shapes()
    assert len(shapes) == 36 * 7 + 1
    weights = sum(N * K for _, _, N, K in shapes)
    assert weights == 7_568_097_280
    assert R.Q4_BYTES_PER_WEIGHT * weights == 4_257_054_720
    total = R.decode_step_bytes(shapes)
    assert total == 4_262_822_656
    assert R.decode_tok_per_s(8000, total) == pytest.approx(1876.7, abs=0.1)


def test_config_byte_counts():
    assert R.q4_gemm_bytes(1, 4096, 4096) == 9_453_568
    assert R.q8_gemm_bytes(16, 12288, 4096, out_bytes=2) == 1.0625 * 12288 * 4096 + 16 * 4096 + 64 + 2 * 16 * 12288
    assert R.moe_token_bytes(16, 7168, 2048) == 16 * 23_396_352 + 4 * 7168 + 8 * 16 * 2048
