// gemm_i8.hip -- int8 x int8 -> int32 GEMM on the gfx950 matrix cores with
// the fused dequant + bias epilogue of the ConvRot linear layer.
//
// What is computed (page "int8 Compute", InvokeAI docs, opening section: the
// layer multiplies int8 by int8 on the int8 matrix units; "What stays on the
// default path": outputs in BF16):
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]                 (int32, exact)
//   y[m][n]   = bf16_rne(fmaf((float)acc, x_scale[m] * w_scale, bias[n]))
//
// Design for CDNA4:
//  * v_mfma_i32_16x16x64_i8.  The weight tile is the instruction's A operand
//    and the activation tile its B operand, so the 16x16 result block of a
//    lane holds four consecutive output channels n of one token m: the
//    epilogue stores 4 bf16 (8 bytes) per lane with no transpose.
//  * Both operands are K-contiguous in HBM ([N, K] weight as stored by
//    nn.Linear, [M, K] codes), so an A or B fragment is 16 rows x 16
//    consecutive bytes: one ds_read_b128 per lane.  Which bytes of a 64-byte k
//    step a lane supplies does not matter for an integer dot product as long
//    as both operands use the same mapping, and they do.
//  * Global -> register -> LDS staging with two LDS stages: the next k-slab
//    is fetched while the MFMAs run on the current one; one barrier per slab.
//    LDS rows are BK bytes; 16-byte chunks are XOR-swizzled by row so that
//    the 16 rows read by one ds_read_b128 hit distinct banks.
//  * Tile order: the dispatcher places workgroup i on XCD i % 8, so the
//    workgroup id is remapped to give each XCD a contiguous run of tiles, and
//    runs are walked in groups of kGroupM token tiles so that neighbouring
//    tiles of one XCD share weight and activation rows in its L2.
//  * Ragged edges: rows past M or N are loaded from the last valid row (the
//    results are discarded) and stores are masked; K is a multiple of 128.
#include "convrot_internal.hpp"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int BN_, int BM_, int BK_, int WN_, int WM_, int SWZ_SHIFT_, int GROUP_M_>
struct Tile {
  static constexpr int BN = BN_;          // output channels per workgroup
  static constexpr int BM = BM_;          // tokens per workgroup
  static constexpr int BK = BK_;          // bytes of K per LDS stage
  static constexpr int WN = WN_;          // waves along n
  static constexpr int WM = WM_;          // waves along m
  static constexpr int kSwzShift = SWZ_SHIFT_;
  static constexpr int kGroupM = GROUP_M_;
  static constexpr int kThreads = WN * WM * 64;
  static constexpr int kWaveN = BN / WN, kWaveM = BM / WM;
  static constexpr int TN = kWaveN / 16, TM = kWaveM / 16;
  static constexpr int kCpr = BK / 16;                       // 16-byte chunks per LDS row
  static constexpr int kALoads = BN * kCpr / kThreads;
  static constexpr int kBLoads = BM * kCpr / kThreads;
  static constexpr int kStageBytes = (BN + BM) * BK;
  static_assert(BN % (WN * 16) == 0 && BM % (WM * 16) == 0, "wave tile");
  static_assert(BK % 64 == 0, "k step");
  static_assert((BN * kCpr) % kThreads == 0 && (BM * kCpr) % kThreads == 0, "loads");
};

// 256 x 256 tokens x channels, 8 waves (each 128 channels x 64 tokens).
using TileBig = Tile<256, 256, 128, 2, 4, 0, 4>;
// 128 x 128, 4 waves (each 64 x 64) for layers too small to fill the chip.
using TileMid = Tile<128, 128, 128, 2, 2, 0, 4>;

template <class T>
__device__ inline int swizzle(int row, int chunk) {
  return chunk ^ ((row >> T::kSwzShift) & (T::kCpr - 1));
}

// Workgroup id -> (channel tile, token tile).
template <class T>
__device__ inline void tile_coords(int tiles_n, int tiles_m, int& tn, int& tm) {
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  {  // contiguous tile runs per XCD
    const int q = nb >> 3, r = nb & 7;
    const int x = bid & 7, local = bid >> 3;
    bid = x * q + (x < r ? x : r) + local;
  }
  const int per_group = T::kGroupM * tiles_n;
  const int gid = bid / per_group;
  const int first_m = gid * T::kGroupM;
  const int gsz = min(tiles_m - first_m, T::kGroupM);
  const int in_group = bid - gid * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = static_cast<__bf16>(a);   // v_cvt_pk_bf16_f32: round to nearest even
  const __bf16 hb = static_cast<__bf16>(b);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

template <class T, bool DEQUANT>
__global__ __launch_bounds__(T::kThreads) void gemm_i8_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    int tiles_n, int tiles_m, const float* __restrict__ x_scale,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  __shared__ uint4 lds[2 * T::kStageBytes / 16];

  int tn, tm;
  tile_coords<T>(tiles_n, tiles_m, tn, tm);
  const int n0 = tn * T::BN, m0 = tm * T::BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / T::WM, wm = wave % T::WM;

  // per-thread global sources and LDS destinations of the staged chunks
  const int8_t* a_src[T::kALoads];
  const int8_t* b_src[T::kBLoads];
  int a_dst[T::kALoads], b_dst[T::kBLoads];
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) {
    const int ch = tid + i * T::kThreads;
    const int r = ch / T::kCpr, c = ch % T::kCpr;
    const int g = min(n0 + r, N - 1);
    a_src[i] = wq + static_cast<int64_t>(g) * K + c * 16;
    a_dst[i] = (r * T::BK) / 16 + swizzle<T>(r, c);
  }
#pragma unroll
  for (int i = 0; i < T::kBLoads; ++i) {
    const int ch = tid + i * T::kThreads;
    const int r = ch / T::kCpr, c = ch % T::kCpr;
    const int g = min(m0 + r, M - 1);
    b_src[i] = xq + static_cast<int64_t>(g) * K + c * 16;
    b_dst[i] = (T::BN * T::BK + r * T::BK) / 16 + swizzle<T>(r, c);
  }

  // LDS fragment offsets (in uint4 units) for k step 0 of a stage
  const int frag_row = lane & 15, frag_chunk = lane >> 4;
  int a_frag[T::TN], b_frag[T::TM];
#pragma unroll
  for (int t = 0; t < T::TN; ++t) {
    const int r = wn * T::kWaveN + t * 16 + frag_row;
    a_frag[t] = r * T::kCpr;
  }
#pragma unroll
  for (int t = 0; t < T::TM; ++t) {
    const int r = wm * T::kWaveM + t * 16 + frag_row;
    b_frag[t] = (T::BN * T::BK) / 16 + r * T::kCpr;
  }

  v4i acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  uint4 ra[T::kALoads], rb[T::kBLoads];
  const int KT = K / T::BK;

  // prologue: slab 0 -> stage 0
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
#pragma unroll
  for (int i = 0; i < T::kBLoads; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
#pragma unroll
  for (int i = 0; i < T::kALoads; ++i) lds[a_dst[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < T::kBLoads; ++i) lds[b_dst[i]] = rb[i];
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int stage = (kt & 1) * (T::kStageBytes / 16);
    // fetch slab kt+1 (the last iteration re-fetches its own slab into the
    // stage nobody reads any more, which keeps the loop free of branches)
    const int64_t k0 = static_cast<int64_t>(kt + 1 < KT ? kt + 1 : kt) * T::BK;
#pragma unroll
    for (int i = 0; i < T::kALoads; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < T::kBLoads; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
#pragma unroll
    for (int kk = 0; kk < T::BK / 64; ++kk) {
      v4i af[T::TN], bf[T::TM];
#pragma unroll
      for (int t = 0; t < T::TN; ++t) {
        const int r = wn * T::kWaveN + t * 16 + frag_row;
        af[t] = __builtin_bit_cast(v4i, lds[stage + a_frag[t] + swizzle<T>(r, kk * 4 + frag_chunk)]);
      }
#pragma unroll
      for (int t = 0; t < T::TM; ++t) {
        const int r = wm * T::kWaveM + t * 16 + frag_row;
        bf[t] = __builtin_bit_cast(v4i, lds[stage + b_frag[t] + swizzle<T>(r, kk * 4 + frag_chunk)]);
      }
#pragma unroll
      for (int i = 0; i < T::TN; ++i)
#pragma unroll
        for (int j = 0; j < T::TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    const int next = (T::kStageBytes / 16) - stage;
#pragma unroll
    for (int i = 0; i < T::kALoads; ++i) lds[next + a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < T::kBLoads; ++i) lds[next + b_dst[i]] = rb[i];
    __syncthreads();
  }

  // epilogue: lane holds acc[i][j][e] = D[n = n0 + wn*kWaveN + i*16 + 4*(lane/16) + e]
  //                                       [m = m0 + wm*kWaveM + j*16 + lane%16]
  const int n_lane = n0 + wn * T::kWaveN + 4 * (lane >> 4);
  const int m_lane = m0 + wm * T::kWaveM + (lane & 15);
  const bool vec = (N & 3) == 0;
  if constexpr (DEQUANT) {
    uint16_t* y = static_cast<uint16_t*>(out);
    const float sw = *w_scale;
    float alpha[T::TM];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) {
      const int m = m_lane + j * 16;
      alpha[j] = m < M ? x_scale[m] * sw : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      const int n = n_lane + i * 16;
      float b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = (bias != nullptr && n + e < N) ? bf16_to_f32(bias[n + e]) : 0.0f;
#pragma unroll
      for (int j = 0; j < T::TM; ++j) {
        const int m = m_lane + j * 16;
        if (m >= M) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(static_cast<float>(acc[i][j][e]), alpha[j], b[e]);
        uint16_t* dst = y + static_cast<int64_t>(m) * N + n;
        if (vec && n + 3 < N) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = static_cast<uint16_t>(pack_bf16x2(v[e], 0.0f) & 0xffffu);
        }
      }
    }
  } else {
    int32_t* c = static_cast<int32_t*>(out);
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      const int n = n_lane + i * 16;
#pragma unroll
      for (int j = 0; j < T::TM; ++j) {
        const int m = m_lane + j * 16;
        if (m >= M) continue;
        int32_t* dst = c + static_cast<int64_t>(m) * N + n;
        if (vec && n + 3 < N) {
          *reinterpret_cast<int4*>(dst) = make_int4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = acc[i][j][e];
        }
      }
    }
  }
}

template <class T, bool DEQUANT>
hipError_t launch_tile(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, const uint16_t* bias, void* out, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_n = static_cast<int>((N + T::BN - 1) / T::BN);
  const int tiles_m = static_cast<int>((M + T::BM - 1) / T::BM);
  const int64_t blocks = static_cast<int64_t>(tiles_n) * tiles_m;
  hipLaunchKernelGGL((gemm_i8_kernel<T, DEQUANT>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(T::kThreads), 0, stream, wq, xq, static_cast<int>(M), static_cast<int>(N),
                     static_cast<int>(K), tiles_n, tiles_m, x_scale, w_scale, bias, out);
  return hipGetLastError();
}

// Pick the tile: the large one when it still gives every CU a few tiles.
template <bool DEQUANT>
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, const uint16_t* bias, void* out, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 512)
    return launch_tile<TileBig, DEQUANT>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  return launch_tile<TileMid, DEQUANT>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
}

}  // namespace

hipError_t launch_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const uint16_t* bias, uint16_t* y,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return launch_gemm<true>(xq, x_scale, wq, w_scale, bias, y, M, N, K, stream);
}

hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M,
                           int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return launch_gemm<false>(xq, nullptr, wq, nullptr, nullptr, acc, M, N, K, stream);
}

}  // namespace convrot
