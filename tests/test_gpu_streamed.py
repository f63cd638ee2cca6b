"""Layers whose int8 weights stay in pinned host memory (page "int8 Compute",
"Partially loaded models": the int8 weight of such a layer crosses to the GPU
on every step and the layer's result does not change by a bit).

convrot_linear_streamed copies each weight into one of two device slots on a
copy stream while the previous layer computes.  Every output must equal, byte
for byte, convrot_linear with the weight resident on the device, and, on
seeded token rows, the CPU oracle's layer computed from the same fp32 weight
(its own weight preparation, rotation, quantization, integer product and
epilogue).  The layer sequence mixes shapes (so slot reuse crosses sizes) and
repeats a weight.
"""
import numpy as np
import pytest

import oracle
from tests._util import bits_of, same_bf16

pytestmark = pytest.mark.gpu


def make_layers(torch, B, synth, shapes, M, seed):
    r = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    out = []
    for i, (K, N) in enumerate(shapes):
        w_np = (r.standard_normal((N, K)) * 0.02).astype(np.float32)
        wq, s_w = B.convrot_prepare_weight(torch.from_numpy(w_np).to(dev), 128)
        x_bits = synth.to_bf16_bits(r.standard_t(4, (M, K)))
        x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        b_bits = synth.to_bf16_bits(r.standard_normal(N) * 0.01)
        bias = torch.from_numpy(b_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        out.append({"x": x, "wq": wq, "wq_host": wq.cpu().pin_memory(), "w_scale": s_w, "group": 128,
                    "bias": bias if i % 3 else None,
                    "_w": w_np, "_x_bits": x_bits, "_b_bits": b_bits if i % 3 else None})
    return out


@pytest.mark.parametrize("created_streams", [False, True])
@pytest.mark.parametrize("M", [16, 700])
def test_streamed_layers_match_resident(M, created_streams):
    # on created streams the copies really overlap the compute (the null
    # stream serialises them), so slot reuse across steps is exercised
    import torch
    from w8a8_rotated_int8_convrot_amd import binding as B, synth
    shapes = [(1024, 3072), (3072, 1024), (1024, 4096), (4096, 1024), (1024, 3072), (2048, 2048)]
    layers = make_layers(torch, B, synth, shapes, M, M)
    layers.append(dict(layers[1]))                              # the same weight again
    resident = [B.convrot_linear(L["x"], L["wq"], L["w_scale"], L["group"], L["bias"]) for L in layers]
    torch.cuda.synchronize()
    for L in layers:
        L["out"] = None
    if created_streams:
        comp = torch.cuda.Stream()
        comp.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(comp):
            for _ in range(3):            # repeated calls reuse the slots back to back
                outs = B.convrot_linear_streamed(layers, copy_stream=torch.cuda.Stream())
    else:
        outs = B.convrot_linear_streamed(layers)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, resident)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"layer {i}"
    # against the oracle: its own prepared weight, the layer on seeded rows
    for i, (L, a) in enumerate(zip(layers, outs)):
        wq_ref, s_ref = oracle.quant_weight(L["_w"], 128)
        rows = np.arange(M) if M <= 32 else synth.sample_rows(M, 24, 100 + i)
        y_ref, _, _ = oracle.linear_rows(L["_x_bits"], rows, wq_ref, s_ref, 128, L["_b_bits"])
        got = bits_of(a[torch.from_numpy(rows).to(a.device)])
        assert np.all(same_bf16(got, y_ref)), f"layer {i} differs from the oracle"


def test_streamed_refuses_pageable_weights():
    import torch
    from w8a8_rotated_int8_convrot_amd import binding as B, synth
    layers = make_layers(torch, B, synth, [(1024, 1024)], 32, 3)
    layers[0]["wq_host"] = layers[0]["wq"].cpu()                 # not pinned
    with pytest.raises(B.ConvrotError) as e:
        B.convrot_linear_streamed(layers)
    assert "pinned" in str(e.value)
