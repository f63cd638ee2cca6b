// convrot_internal.hpp -- shared declarations of the HIP library (not part of
// the C ABI).  Kernels live in rotate_quant.hip (rotation + quantization, and
// the default path's weight unpacking), gemm_i8.hip (the int8 GEMM with its
// epilogues, and the default path's bf16/fp16 product on the same tiles),
// default_path.hip (the guarded layer's check) and mfma_probe.hip (two
// measurement aids); argument checking, dispatch and the guard state live in
// convrot_api.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace convrot {

// Largest K the library accepts: 127 * 127 * K must stay below 2^31 so that
// an int32 accumulator cannot overflow.
constexpr int64_t kMaxK = 131072;

// Compute units of the current device (read once; 256 on MI355X), which the
// launch shapes are balanced over.
int num_cus();

// ---------------------------------------------------------------- rotate + quant

// Per-token rotate + quantize of a bf16 [M, K] activation into int8 codes and
// fp32 scales.  group is 128 or 256; K % group == 0.
hipError_t launch_rotate_quant(const uint16_t* x, int64_t M, int64_t K, int group,
                               int8_t* q, float* scale, hipStream_t stream);
// The same for an IEEE binary16 activation (bits passed as uint16_t).
hipError_t launch_rotate_quant_f16(const uint16_t* x, int64_t M, int64_t K, int group,
                                   int8_t* q, float* scale, hipStream_t stream);

// Weight preparation.  in_dtype: kInF32, kInBf16 or kInF16.  Tensorwise (one
// scale; `amax_cell` is one 4-byte device word of scratch) or, with
// row_scale, one scale per output channel (w_scale [N]; no scratch).
constexpr int kInF32 = 0, kInBf16 = 1, kInF16 = 2;
hipError_t launch_prepare_weight(const void* w, int in_dtype, bool row_scale, int64_t N, int64_t K,
                                 int group, int8_t* wq, float* w_scale, uint32_t* amax_cell,
                                 hipStream_t stream);

// Default path: unpack a rotated int8 weight, out[n] = rnd(rotate(s * wq[n]))
// (s = w_scale[row_scale ? n : 0]), rnd = bf16 or fp16 (out_f16) RNE.
hipError_t launch_unpack_weight(const int8_t* wq, const float* w_scale, bool row_scale, int64_t N,
                                int64_t K, int group, bool out_f16, uint16_t* out, hipStream_t stream);

// ---------------------------------------------------------------- GEMM

// GEMM + fused dequant/bias epilogue: y[m][n] (bf16) from xq [M, K] and
// wq [N, K].  K % 128 == 0.
hipError_t launch_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const uint16_t* bias, uint16_t* y,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Variants: one weight scale per output channel (row_scale: w_scale [N]) and
// fp16 in place of bf16 for the bias and the output (out_f16).
hipError_t launch_gemm_dequant_ex(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, bool row_scale, const uint16_t* bias,
                                  uint16_t* y, bool out_f16, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream);

// Same main loop with the raw int32 products stored.
hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Default path product: y = rnd(x . wu^T + bias) on bf16 (or fp16, f16)
// operands x [M, K] and wu [N, K] with an fp32 accumulator.  K % 64 == 0.
hipError_t launch_gemm_default(const uint16_t* x, const uint16_t* wu, const uint16_t* bias, uint16_t* y,
                               bool f16, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// ---------------------------------------------------------------- guard check
// (default_path.hip)

// xs[i] = x[row_i] for the R sampled rows row_i = i * (M - 1) / (R - 1).
hipError_t launch_gather_rows(const uint16_t* x, int64_t M, int64_t K, int R, uint16_t* xs,
                              hipStream_t stream);
// Per sampled row i: partial[3i..3i+2] = {sum_n (a - b)^2, sum_n b^2, count of
// mismatched non-finite values}, a = y[row_i][n] (negated when flip),
// b = ydef[i][n], in fp64; where a and b are the same infinity the position
// is left out of the sums, and where either is otherwise not finite it counts.
hipError_t launch_compare_rows(const uint16_t* y, const uint16_t* ydef, bool f16, int64_t M, int64_t N,
                               int R, bool flip, double* partial, hipStream_t stream);
// The sampled row i of R over M rows.
__host__ __device__ inline int64_t sample_row(int i, int R, int64_t M) {
  return R > 1 ? static_cast<int64_t>(i) * (M - 1) / (R - 1) : 0;
}

// ---------------------------------------------------------------- measurement aid

// Register-only MFMA loop (mfma_probe.hip): `blocks` workgroups of 256
// threads, `iters` x 16 v_mfma_i32_32x32x32_i8 per wave on 16-byte fragments
// taken from a and b; one int32 per thread written to out.
hipError_t launch_mfma_probe(const int8_t* a, int64_t a_bytes, const int8_t* b, int64_t b_bytes,
                             int blocks, int iters, int32_t* out, hipStream_t stream);
// Plain stream (mfma_probe.hip): q[i] = high byte of x[i] for n 16-bit
// values (n % 8 == 0, 16-byte aligned buffers).
hipError_t launch_stream_probe(const uint16_t* x, int64_t n, int8_t* q, hipStream_t stream);

}  // namespace convrot
