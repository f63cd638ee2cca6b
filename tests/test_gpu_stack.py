"""The benchmark's DiT denoising-step stack checked against the oracle.

The stack's weights, biases and token rows are drawn on the device by a seeded
torch generator (synth.stack_weight_device, synth.stack_tokens_device), exactly
as the benchmark draws them.  For blocks 0 and 59 every layer runs through the
C ABI as the benchmark runs it: QKV and MLP-up on the block input, the
out-projection on the attention-output stand-in, MLP-down on the MLP-up
output.  The oracle takes the host copies of the same weights and token rows,
prepares the weights itself, and evaluates each layer on seeded token rows;
its down layer reads its own up layer's output for those rows.  Every token
is rotated and quantized on its own, so a sampled row of a layer is exactly
that row of the full layer, and the comparison is bit for bit (the up layer's
rows agree bit for bit, so the down layer's inputs do too).
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bits_of
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from w8a8_rotated_int8_convrot_amd import binding
    binding.lib()
    return binding


@pytest.mark.parametrize("block", [0, 59])
def test_stack_block_against_oracle(B, block):
    g = 128
    x_in = synth.stack_tokens_device(1, DEV)
    x_attn = synth.stack_tokens_device(2, DEV)
    xin_bits = bits_of(x_in)
    xattn_bits = bits_of(x_attn)
    # every token row's absmax lies in [5, 30] (before the bf16 rounding)
    amax = np.abs(oracle.bf16_bits_to_f32(xin_bits)).max(axis=1)
    assert amax.min() >= 4.9 and amax.max() <= 30.2
    rows = synth.sample_rows(synth.STACK_M, 24, 0x57AC + block)
    ridx = torch.from_numpy(rows).to(DEV)
    y_gpu, y_ref = {}, {}
    for li, (kind, K, N) in enumerate(synth.STACK_LAYERS):
        w, bias = synth.stack_weight_device(block, li, DEV)
        wq, s_w = B.convrot_prepare_weight(w, g)
        x = {"qkv": x_in, "out": x_attn, "up": x_in, "down": None}[kind]
        if kind == "down":
            x = y_gpu["up"]
        y = B.convrot_linear(x, wq, s_w, g, bias)
        torch.cuda.synchronize()
        y_gpu[kind] = y
        # the oracle's own weight preparation from the host copy of the weight
        w_host = w.cpu().numpy()
        b_bits = bits_of(bias)
        wq_ref, s_ref = oracle.quant_weight(w_host, g)
        assert np.array_equal(wq.cpu().numpy(), wq_ref), kind
        assert s_w.item() == float(s_ref), kind
        if kind == "down":
            # the oracle's down layer on its own up layer's rows
            yr, _, _ = oracle.linear_rows(y_ref["up"], np.arange(len(rows)), wq_ref, s_ref, g, b_bits)
        else:
            xb = xattn_bits if kind == "out" else xin_bits
            yr, _, _ = oracle.linear_rows(xb, rows, wq_ref, s_ref, g, b_bits)
        y_ref[kind] = yr
        got = bits_of(y[ridx])
        assert np.array_equal(got, yr), f"block {block} {kind}: {int(np.sum(got != yr))} outputs differ"
