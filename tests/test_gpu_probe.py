"""The measurement aids of the benchmark (not steps of the layer) do what they
claim.  The MFMA-rate probe really runs its int8 products on the operand bytes
it is given; the plain stream writes the high byte of every 16-bit value.

Each lane of a wave holds four A and four B fragments of 16 bytes and the wave
issues, per iteration, one 16x16x64 int8 MFMA for each of the 16 (A, B)
pairs.  Summed over the whole 16x16 result, an MFMA gives
sum_k colsum_A[k] * colsum_B[k], where the column sums run over the 16 lanes
that share a quarter of K; that total does not depend on how the instruction
maps a lane's bytes to k, as long as A and B use the same mapping.  So the sum
of a wave's per-lane checksums is iters * sum over the 16 pairs of those
totals, computed here in int64 from the same bytes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def expected_wave_sums(a, b, blocks, iters):
    a_chunks, b_chunks = a.size // 16, b.size // 16
    out = []
    for w in range(blocks * 12):
        t = np.arange(w * 64, w * 64 + 64)
        fa = [a.reshape(-1, 16)[(t * 4 + i) % a_chunks].astype(np.int64) for i in range(4)]
        fb = [b.reshape(-1, 16)[(t * 4 + i) % b_chunks].astype(np.int64) for i in range(4)]
        total = 0
        for i in range(16):
            A, B = fa[i & 3], fb[i >> 2]
            for h in range(4):
                total += int((A[h * 16:h * 16 + 16].sum(0) * B[h * 16:h * 16 + 16].sum(0)).sum())
        out.append(iters * total)
    return np.array(out, dtype=np.int64)


@pytest.mark.parametrize("a_bytes,b_bytes,blocks,iters", [(4096, 8192, 2, 3), (1 << 16, 208, 3, 5)])
def test_probe_checksums(a_bytes, b_bytes, blocks, iters):
    import torch
    from w8a8_rotated_int8_convrot_amd import binding
    rng = np.random.default_rng(7)
    a = rng.integers(-127, 128, a_bytes, dtype=np.int8)
    b = rng.integers(-127, 128, b_bytes, dtype=np.int8)
    out = binding.convrot_probe_mfma_i8(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                                        blocks, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(blocks * 12, 64).sum(1)
    np.testing.assert_array_equal(got, expected_wave_sums(a, b, blocks, iters))


@pytest.mark.parametrize("n", [8, 8000, 2048 * 256 * 8 * 3 + 24])
def test_stream_probe_writes_high_bytes(n):
    # the last size makes the 2048 workgroups loop three times and then some
    import torch
    from w8a8_rotated_int8_convrot_amd import binding
    x = np.random.default_rng(n).integers(-32768, 32768, n, dtype=np.int64).astype(np.int16)
    q = binding.convrot_probe_stream(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), (x >> 8).astype(np.int8))
