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
//    and the activation tile its B operand, so a lane's 16x16 result block
//    holds four consecutive output channels n of one token m.
//  * Both operands are K-contiguous in HBM ([N, K] weight as stored by
//    nn.Linear, [M, K] codes), so an A or B fragment is 16 rows x 16
//    consecutive bytes: one ds_read_b128 per lane.  Which bytes of a 64-byte k
//    step a lane supplies does not matter for an integer dot product as long
//    as both operands use the same mapping, and they do.
//  * Global -> LDS by direct-to-LDS loads (global_load_lds_dwordx4: each
//    wave instruction fills 1 KB = 16 LDS rows of 64 bytes, no registers
//    involved), four LDS stages of one 64-byte k slab each, prefetched three
//    slabs ahead.  A slab is consumed after `s_waitcnt vmcnt` (this wave's
//    loads of that slab have landed) and one `s_barrier` (so have everyone
//    else's, and everyone is done with the stage about to be refilled).
//  * LDS rows are 64 bytes; the four 16-byte chunks of row r are stored XOR
//    (r >> 1) & 3, so the 8 rows served together by one ds_read_b128 pass
//    fall into distinct banks.  A lane's direct-to-LDS slot is fixed by its
//    lane id, so the swizzle is applied by choosing which global chunk the
//    lane fetches.
//  * Epilogue: dequant + bias in registers, bf16 tile staged through LDS
//    (chunk-XOR-swizzled rows), then written out as full contiguous rows with
//    16-byte stores, so every output line leaves the CU whole.
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
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void glb_void_t;

constexpr int kBK = 64;        // bytes of K per LDS stage (one MFMA k step)
constexpr int kStages = 4;     // LDS stages; slabs are prefetched kStages-1 ahead

template <int BN_, int BM_, int WN_, int WM_, int GROUP_M_>
struct Tile {
  static constexpr int BN = BN_;          // output channels per workgroup
  static constexpr int BM = BM_;          // tokens per workgroup
  static constexpr int WN = WN_;          // waves along n
  static constexpr int WM = WM_;          // waves along m
  static constexpr int kGroupM = GROUP_M_;
  static constexpr int kWaves = WN * WM;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWaveN = BN / WN, kWaveM = BM / WM;
  static constexpr int TN = kWaveN / 16, TM = kWaveM / 16;
  static constexpr int kStageBytes = (BN + BM) * kBK;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  // direct-to-LDS instructions per wave and slab (each moves 16 rows)
  static constexpr int kALoads = BN / 16 / kWaves;
  static constexpr int kBLoads = BM / 16 / kWaves;
  static constexpr int kLoads = kALoads + kBLoads;
  static_assert(BN % (WN * 16) == 0 && BM % (WM * 16) == 0, "wave tile");
  static_assert(kALoads * kWaves * 16 == BN && kBLoads * kWaves * 16 == BM, "load split");
  static_assert(BM * BN * 2 <= kLdsBytes, "bf16 output tile must fit the LDS stages");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

// 256 channels x 256 tokens, 8 waves (each 128 channels x 64 tokens).
using TileBig = Tile<256, 256, 2, 4, 4>;
// 128 x 128, 4 waves (each 64 x 64) for layers too small to fill the chip.
using TileMid = Tile<128, 128, 2, 2, 4>;

// s_waitcnt vmcnt(N) + s_barrier.  lgkmcnt(0) too, so that this wave's LDS
// reads of the previous slab are complete before anyone refills its stage.
// The memory clobber keeps every load and store on its side of the barrier.
template <int N>
__device__ inline void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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

// Byte offset of element (row m, column n) of the bf16 output tile staged in
// LDS: rows of BN*2 bytes, 16-byte chunks XOR-swizzled by the row.
template <class T>
__device__ inline int out_lds_offset(int m, int n) {
  constexpr int kChunks = T::BN / 8;
  return m * (T::BN * 2) + ((((n >> 3) ^ m) & (kChunks - 1)) << 4) + ((n & 7) << 1);
}

template <class T, bool DEQUANT>
__global__ __launch_bounds__(T::kThreads) void gemm_i8_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    int tiles_n, int tiles_m, const float* __restrict__ x_scale,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];

  int tn, tm;
  tile_coords<T>(tiles_n, tiles_m, tn, tm);
  const int n0 = tn * T::BN, m0 = tm * T::BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / T::WM, wm = wave % T::WM;

  // ---- direct-to-LDS sources: instruction j of this wave fills LDS rows
  // [16*i, 16*i + 16) of its operand (i = wave * loads + j); lane L lands in
  // row 16*i + L/4, stored chunk L%4, and so fetches global chunk
  // (L%4) ^ ((row >> 1) & 3) of that row.
  const int8_t* src[T::kLoads];
  int dst[T::kLoads];
#pragma unroll
  for (int j = 0; j < T::kLoads; ++j) {
    const bool is_a = j < T::kALoads;
    const int i = is_a ? wave * T::kALoads + j : wave * T::kBLoads + (j - T::kALoads);
    const int row = 16 * i + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 1) & 3);
    if (is_a) {
      src[j] = wq + static_cast<int64_t>(min(n0 + row, N - 1)) * K + chunk * 16;
      dst[j] = i * 16 * kBK;
    } else {
      src[j] = xq + static_cast<int64_t>(min(m0 + row, M - 1)) * K + chunk * 16;
      dst[j] = T::BN * kBK + i * 16 * kBK;
    }
  }
  const int KT = K / kBK;

  auto issue_slab = [&](int slab, int stage) {
    const int64_t k0 = static_cast<int64_t>(slab) * kBK;
#pragma unroll
    for (int j = 0; j < T::kLoads; ++j) {
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src[j] + k0),
                                       (lds_void_t*)(lds + stage * T::kStageBytes + dst[j]),
                                       16, 0, 0);
    }
  };

  // ---- fragment reads: lane reads row (l & 15) of a 16-row block, chunk l >> 4
  const int frag = (lane & 15) * kBK + ((((lane >> 4) ^ ((lane >> 1) & 3)) & 3) << 4);
  const int a_base = wn * T::kWaveN * kBK + frag;
  const int b_base = T::BN * kBK + wm * T::kWaveM * kBK + frag;

  v4i acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue_slab(min(s, KT - 1), s);

  for (int kt = 0; kt < KT; ++kt) {
    // slabs kt+1 .. kt+kStages-2 may still be in flight
    wait_vm_barrier<(kStages - 2) * T::kLoads>();
    // refill the stage consumed in the previous iteration (slab indices past
    // the end re-fetch the last slab into a stage that is never read again)
    issue_slab(min(kt + kStages - 1, KT - 1), (kt + kStages - 1) % kStages);

    const char* st = lds + (kt % kStages) * T::kStageBytes;
    v4i af[T::TN], bf[T::TM];
#pragma unroll
    for (int t = 0; t < T::TN; ++t) af[t] = *reinterpret_cast<const v4i*>(st + a_base + t * 16 * kBK);
#pragma unroll
    for (int t = 0; t < T::TM; ++t) bf[t] = *reinterpret_cast<const v4i*>(st + b_base + t * 16 * kBK);
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
      for (int j = 0; j < T::TM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  }

  // lane holds acc[i][j][e] = D[n = n0 + wn*kWaveN + i*16 + 4*(lane/16) + e]
  //                             [m = m0 + wm*kWaveM + j*16 + lane%16]
  const int n_loc = wn * T::kWaveN + 4 * (lane >> 4);
  const int m_loc = wm * T::kWaveM + (lane & 15);

  if constexpr (DEQUANT) {
    uint16_t* y = static_cast<uint16_t*>(out);
    const float sw = *w_scale;
    float alpha[T::TM];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) {
      const int m = m0 + m_loc + j * 16;
      alpha[j] = x_scale[min(m, M - 1)] * sw;
    }
    // every wave is done with the stages (and every load has landed) before
    // the output tile overwrites them
    wait_vm_barrier<0>();
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      const int nl = n_loc + i * 16;
      float b[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = min(n0 + nl + e, N - 1);
        b[e] = bias != nullptr ? bf16_to_f32(bias[n]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < T::TM; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(static_cast<float>(acc[i][j][e]), alpha[j], b[e]);
        *reinterpret_cast<uint2*>(lds + out_lds_offset<T>(m_loc + j * 16, nl)) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    __syncthreads();
    // full rows out: a row is BN/8 16-byte chunks
    constexpr int kChunks = T::BN / 8;
    constexpr int kRowsPerPass = T::kThreads / kChunks;
    const int ch = tid % kChunks;
    const int n = n0 + ch * 8;
    const bool vec = (N & 7) == 0;
#pragma unroll 4
    for (int r = tid / kChunks; r < T::BM; r += kRowsPerPass) {
      const int m = m0 + r;
      if (m >= M) break;
      const uint4 v = *reinterpret_cast<const uint4*>(lds + out_lds_offset<T>(r, ch * 8));
      uint16_t* dstp = y + static_cast<int64_t>(m) * N + n;
      if (vec && n + 8 <= N) {
        *reinterpret_cast<uint4*>(dstp) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) dstp[e] = static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
    int32_t* c = static_cast<int32_t*>(out);
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      const int n = n0 + n_loc + i * 16;
#pragma unroll
      for (int j = 0; j < T::TM; ++j) {
        const int m = m0 + m_loc + j * 16;
        if (m >= M) continue;
        int32_t* dstp = c + static_cast<int64_t>(m) * N + n;
        if (vec && n + 3 < N) {
          *reinterpret_cast<int4*>(dstp) = make_int4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dstp[e] = acc[i][j][e];
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
