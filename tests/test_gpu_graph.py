"""The layer inside a captured HIP graph.

convrot_linear allocates nothing, synchronises nothing and records no memset,
so a caller can capture it once and replay it.  Every replay here is checked
byte for byte against an eager call on the same input, with fresh input bytes
copied in and other eager work (and synchronisation) between the replays.
Both activation kernels are covered: the row kernel (512 x 3072 = 1.6M
elements) and the block kernel (1024 x 3072).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [512, 1024])
def test_linear_graph_replays_match_eager(M):
    import torch
    from w8a8_rotated_int8_convrot_amd import binding, synth
    dev = torch.device("cuda:0")
    K, N, g = 3072, 1024, 128
    r = np.random.default_rng(M)
    w = torch.from_numpy((r.standard_normal((N, K)) * 0.02).astype(np.float32)).to(dev)
    wq, s_w = binding.convrot_prepare_weight(w, g)
    bias = torch.from_numpy(synth.to_bf16_bits(r.standard_normal(N) * 0.01).view(np.int16)) \
        .view(torch.bfloat16).to(dev)
    inputs = [torch.from_numpy(synth.to_bf16_bits(r.standard_t(4, (M, K))).view(np.int16))
              .view(torch.bfloat16).to(dev) for _ in range(4)]
    x = inputs[0].clone()
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(binding.convrot_linear_workspace(M, K, N), dtype=torch.uint8, device=dev)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):                      # warm-up outside the capture
        binding.convrot_linear(x, wq, s_w, g, bias, out=y, workspace=ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.convrot_linear(x, wq, s_w, g, bias, out=y, workspace=ws)
    torch.cuda.synchronize()

    for i in (1, 2, 3, 0, 2):
        x.copy_(inputs[i])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ref = binding.convrot_linear(inputs[i], wq, s_w, g, bias)   # eager, own buffers
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay with input {i}"
