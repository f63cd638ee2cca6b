"""The DiT MLP pair at 1024^2 run as a chain: up-projection (4608 x 3072 ->
12288), GELU (tanh form) in bf16, down-projection (12288 -> 3072).

GPU chain: convrot_linear (up) -> torch's bf16 GELU on the device (the
harness's own step, outside the library) -> convrot_linear (down).
Oracle chain, from the same seeded activation and weights, on seeded token
rows: oracle up -> the same GELU formula in fp64 on the oracle's bf16 output,
rounded to bf16 -> oracle down.  Each token is rotated and quantized on its
own in both layers, so a sampled row of the chain is exactly that row of the
full chain.

Bars (the same as for a single layer end to end): the down layer's activation
codes at least 99.9 % identical to the oracle chain's, none off by more than
one; bf16 output within relative Frobenius error 1e-2 of the oracle chain.
The GELU of the two chains may round a few values differently (fp32 on the
device, fp64 here), which is why the codes of the second layer are held to
the end-to-end bar rather than bitwise.  The chain's error against the
unquantized fp64 chain (x W_up^T + b, GELU, . W_down^T + b) is printed and
gated at the 0.05 screening level of the page "INT8 ConvRot on 2xT4
(Turing)" (kernel table).
"""
import numpy as np
import pytest
import torch

import oracle
from tests._util import bits_of, rel_frobenius, to_dev_bf16
from w8a8_rotated_int8_convrot_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gelu_tanh_f64(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from w8a8_rotated_int8_convrot_amd import binding
    binding.lib()
    return binding


@pytest.mark.parametrize("g", [128])
def test_mlp_pair_chain_against_oracle_chain(B, g):
    up = synth.make_layer("mlp_up", g=g)
    down = synth.make_layer("mlp_down", g=g)          # its weight and bias (its x is not used)
    assert (up.N, down.K, down.N) == (12288, 12288, 3072)

    # ---- GPU chain over the whole batch
    x = to_dev_bf16(up.x_bits, DEV)
    wq_u, s_u = B.convrot_prepare_weight(torch.from_numpy(up.w).to(DEV), g)
    wq_d, s_d = B.convrot_prepare_weight(torch.from_numpy(down.w).to(DEV), g)
    b_u, b_d = to_dev_bf16(up.bias_bits, DEV), to_dev_bf16(down.bias_bits, DEV)
    y_up = B.convrot_linear(x, wq_u, s_u, g, b_u)
    h = torch.nn.functional.gelu(y_up, approximate="tanh")     # bf16 in, bf16 out
    y = B.convrot_linear(h, wq_d, s_d, g, b_d)
    q_d, _ = B.convrot_rotate_quant(h, g)
    torch.cuda.synchronize()

    # ---- oracle chain on seeded rows
    wq_u_ref, s_u_ref = oracle.quant_weight(up.w, g)
    wq_d_ref, s_d_ref = oracle.quant_weight(down.w, g)
    assert np.array_equal(wq_u.cpu().numpy(), wq_u_ref) and s_u.item() == float(s_u_ref)
    assert np.array_equal(wq_d.cpu().numpy(), wq_d_ref) and s_d.item() == float(s_d_ref)
    rows = synth.sample_rows(up.M, 64, 0xC3)
    y_up_ref, _, _ = oracle.linear_rows(up.x_bits, rows, wq_u_ref, s_u_ref, g, up.bias_bits)
    h_ref = synth.to_bf16_bits(gelu_tanh_f64(oracle.bf16_bits_to_f32(y_up_ref).astype(np.float64)))
    local = np.arange(len(rows))
    y_ref, q_ref, _ = oracle.linear_rows(h_ref, local, wq_d_ref, s_d_ref, g, down.bias_bits)

    ridx = torch.from_numpy(rows).to(DEV)
    # the up layer alone is bit-exact (its codes are), so the GELU inputs agree
    assert np.array_equal(bits_of(y_up[ridx]), y_up_ref)
    h_gpu = bits_of(h[ridx])
    gelu_same = float(np.mean(h_gpu == h_ref))

    q_gpu = q_d[ridx].cpu().numpy().astype(np.int32)
    dq = np.abs(q_gpu - q_ref.astype(np.int32))
    codes_same = float(np.mean(dq == 0))
    y_gpu = bits_of(y[ridx])
    err = rel_frobenius(y_gpu, y_ref)

    # the unquantized chain in fp64 on the same rows
    up64 = oracle.reference_fp64(up.x_bits[rows], up.w, up.bias_bits)
    h64 = gelu_tanh_f64(up64)
    y64 = h64 @ down.w.astype(np.float64).T + oracle.bf16_bits_to_f32(down.bias_bits).astype(np.float64)
    chained = oracle.nrmse(oracle.bf16_bits_to_f32(y_gpu), y64)
    print(f"\nMLP pair chain, {len(rows)} rows: GELU outputs identical {gelu_same:.6f}; down codes identical "
          f"{codes_same:.6f}, max |dcode| {int(dq.max())}; rel-Frobenius vs oracle chain {err:.3e}; "
          f"chained NRMSE vs unquantized fp64 chain {chained:.4f}", flush=True)

    assert codes_same >= 0.999, codes_same
    assert dq.max() <= 1
    assert err <= 1e-2, err
    assert np.all(np.isfinite(oracle.bf16_bits_to_f32(y_gpu)))
    assert chained <= 0.05, chained
