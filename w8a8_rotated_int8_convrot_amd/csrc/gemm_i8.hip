// gemm_i8.hip -- int8 x int8 -> int32 GEMM on the gfx950 matrix cores with
// the fused dequant + bias epilogue of the ConvRot linear layer.
//
// What is computed (page "int8 Compute", InvokeAI docs, opening section: the
// product of the two code tensors runs on the integer matrix units; "What
// stays on the default path": outputs in BF16):
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]                 (int32, exact)
//   y[m][n]   = bf16_rne(fmaf((float)acc, x_scale[m] * w_scale, bias[n]))
//
// Kernels: gemm_i8_kernel (one tile per workgroup, any tile shape below),
// gemm_persist_kernel (one workgroup per CU walking several 384 x 192 or
// 192 x 288 tiles, its epilogue overlapped with the next tile's first MFMAs)
// and gemm_ksplit_kernel / gemm_ksplit_reg_kernel (at most 16 tokens: the
// four waves of a workgroup split K; the second streams the operands through
// registers, for K = 3072 and 4096).  Which one runs is a performance choice (pick_tile): on the int8
// path every one gives the same bytes (integer sums are exact in any order).
//
// Design for CDNA4:
//  * v_mfma_i32_32x32x32_i8 (v_mfma_i32_16x16x64_i8 in the 8-wave, 192 x 288
//    and small tiles).  The weight tile is the instruction's A operand and
//    the activation tile its B operand, so a lane's result block holds four
//    consecutive output channels n of one token m.
//  * Both operands are K-contiguous in HBM ([N, K] weight as stored by
//    nn.Linear, [M, K] codes), so an A or B fragment is MF rows x 16
//    consecutive bytes: one ds_read_b128 per lane.  Which bytes of a k step
//    a lane supplies does not matter for an integer dot product as long as
//    both operands use the same mapping, and they do.
//  * Global -> LDS by direct-to-LDS loads (global_load_lds_dwordx4: each
//    wave instruction fills 1 KB of LDS rows, no registers involved).  A
//    "slab" is BK bytes of K of both operand tiles.  Two pipelines:
//    - BK = 128, two stages (the 192 x 288, 384 x 192 and 384 x 96 tiles):
//      the slab after next is issued at each slab boundary into the stage
//      just finished; a row's 128 bytes are one request, which halves the
//      L1 -> L2 request count of 64-byte slabs, and there is one barrier per
//      128 bytes of K;
//    - BK = 64 or 128, three or more stages, prefetched kStages-1 slabs
//      ahead (the other tiles; the K-split kernel gives each wave its own
//      two-stage ring).
//    Fragments are double-buffered per MFMA k step: while one k step's MFMAs
//    run from one register set, the LDS reads of the next fill the other.
//    A load's address is a scalar base (the tile's first operand row plus the
//    slab's K offset) and a fixed 32-bit per-lane offset, and its LDS
//    destination (M0) is computed by the scalar unit: nothing on the vector
//    side sits between a slab's loads, so issuing them does not hold up the
//    MFMAs that follow (2-3.5 % faster than 64-bit per-lane addresses
//    rebuilt in one register pair before every load).
//    Stage reuse is guarded by `s_waitcnt vmcnt` (this wave's loads of the
//    needed slab have landed) and one `s_barrier` (so have everyone else's,
//    and everyone is done with the stage about to be refilled).
//  * LDS rows are BK bytes; the 16-byte chunks of a row are stored
//    XOR-swizzled by row bits (swz below), so the lanes served together by
//    one ds_read_b128 pass fall into distinct banks.  A lane's direct-to-LDS
//    slot is fixed by its lane id, so the swizzle is applied by choosing
//    which global chunk the lane fetches.
//  * Epilogue: dequant + bias in registers.  The one-tile kernel stages the
//    bf16 tile through LDS (chunk-XOR-swizzled rows) and writes full
//    contiguous rows with 16-byte stores; the persistent kernel stores
//    straight from registers after a lane exchange (v_permlane32_swap or
//    v_permlane16_swap) that gives each lane 16 contiguous bytes.
//  * Tile order: the dispatcher places workgroup i on XCD i % 8, so the
//    workgroup id is remapped to give each XCD a contiguous run of tiles, and
//    runs are walked in groups of kGroupM token tiles so that neighbouring
//    tiles of one XCD share weight and activation rows in its L2.
//  * Ragged edges: rows past M or N are loaded from the last valid row (the
//    results are discarded) and stores are masked; K is a multiple of 128.
//  * The same kernel runs the default (dequantizing) path's bf16 or fp16
//    product (page "int8 Compute", "When something goes wrong": the guarded
//    layer checks its first result against that path and may fall back to
//    it): a v_mfma_f32_32x32x16_bf16 / _f16 lane takes 8 values = 16 bytes of
//    one row, exactly as an int8 lane takes 16 codes, and the 32x32 result
//    layout is the same, so the tiles are used with K counted in bytes and
//    an fp32 accumulator; the epilogue is rnd(acc + bias).
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "convrot_internal.hpp"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void glb_void_t;

template <int BN_, int BM_, int WN_, int WM_, int MF_, int GROUP_M_, int STAGES_ = 4, int BK_ = 64>
struct Tile {
  static constexpr int kStages = STAGES_;  // LDS stages; slabs are prefetched kStages-1 ahead
  static constexpr int BK = BK_;           // bytes of K per LDS stage (a "slab")
  static constexpr int kRowChunks = BK / 16;       // 16-byte chunks per LDS row
  static constexpr int kRowsPerLoad = 64 / kRowChunks;   // LDS rows one direct-to-LDS instruction fills
  static constexpr int BN = BN_;          // output channels per workgroup
  static constexpr int BM = BM_;          // tokens per workgroup
  static constexpr int WN = WN_;          // waves along n
  static constexpr int WM = WM_;          // waves along m
  static constexpr int MF = MF_;          // MFMA block: 16 (16x16x64) or 32 (32x32x32)
  static constexpr int kGroupM = GROUP_M_;
  static constexpr int kWaves = WN * WM;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWaveN = BN / WN, kWaveM = BM / WM;
  static constexpr int TN = kWaveN / MF, TM = kWaveM / MF;   // MFMA blocks per wave
  static constexpr int kUnitBytes = MF == 16 ? 64 : 32;     // K bytes of one MFMA
  static constexpr int kKSteps = BK / kUnitBytes;            // MFMA k steps per slab
  static constexpr int kAccRegs = MF == 16 ? 4 : 16;
  static constexpr int kStageBytes = (BN + BM) * BK;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  // direct-to-LDS instructions per wave and slab (each moves 16 rows)
  static constexpr int kALoads = BN / kRowsPerLoad / kWaves;
  static constexpr int kBLoads = BM / kRowsPerLoad / kWaves;
  static constexpr int kLoads = kALoads + kBLoads;
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(BN % (WN * MF) == 0 && BM % (WM * MF) == 0, "wave tile");
  static_assert(BK == 64 || BK == 128, "slab width");
  static_assert(kALoads * kWaves * kRowsPerLoad == BN && kBLoads * kWaves * kRowsPerLoad == BM,
                "load split");
  static_assert(BM * BN * 2 <= kLdsBytes, "bf16 output tile must fit the LDS stages");
  static_assert(kThreads % (BN / 8) == 0, "epilogue rows per pass");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  // two stages (double buffering, the slab after next issued at each slab
  // boundary) or three and more (prefetched kStages-1 slabs ahead)
  static_assert(kStages >= 2 && (kStages - 2) * kLoads < 64 && kLoads < 64, "stages / vmcnt range");
};

// 256 channels x 256 tokens, 4 waves (each 128 x 128 with 32x32x32 MFMAs;
// the 256 accumulator registers per lane live in AGPRs).
using TileBig = Tile<256, 256, 2, 2, 32, 4>;
// 256 x 256, 8 waves (each 128 channels x 64 tokens, 16x16x64 MFMAs).
using TileBig8 = Tile<256, 256, 2, 4, 16, 4>;
// 384 channels x 192 tokens, 12 waves (each 96 x 64, 32x32x32 MFMAs, three
// waves per SIMD).  M = 4608, N = 12288 splits into 768 such tiles: exactly
// three rounds over 256 CUs, where 256 x 256 tiles leave the fourth round
// 62 % empty.
using TileWide = Tile<384, 192, 4, 3, 32, 4>;
// 128 x 128, 4 waves (each 64 x 64) for layers too small to fill the chip.
using TileMid = Tile<128, 128, 2, 2, 16, 4>;
// Few tokens (M <= 32): the weight stream is the whole cost.  32 channels x
// 32 tokens per one-wave workgroup, so N/32 workgroups stream disjoint weight
// rows, each with 15 slabs (30 KB) of loads in flight.
using TileSkinny = Tile<32, 32, 1, 1, 32, 1, 16>;
// M <= 16: 16 channels x 16 tokens per one-wave workgroup (16x16x64 MFMAs),
// eight stages of 128-byte slabs (4 KB: every direct-to-LDS load moves eight
// whole 128-byte rows), so that three workgroups share a CU: N = 12288 gives
// 768 workgroups, exactly three per CU.  With the weight read from HBM,
// 16 x 3072 x 12288 takes 13.2 us (16.7 with 24 stages of 64-byte slabs, 12
// stages of 128 bytes 14.2), 16 x 12288 x 4096 12.2 us (13.0; 12.6); with
// many channels the K-split tile below is faster still.
using TileSkinny16 = Tile<16, 16, 1, 1, 16, 1, 8, 128>;
// 384 x 192 as TileWide, but 128-byte slabs in two stages: one barrier per
// 128 bytes of K, and the direct-to-LDS loads fetch 128 contiguous bytes of
// a row (eight lanes) per request instead of 64.  Tiles are walked in groups
// of 8 token tiles, so the 32 tiles one XCD runs at a time are 8 token tiles
// x 4 channel tiles: 9.4 MB of operand panels per round in that XCD's L2
// instead of 11.8 MB with groups of 4 (8 channel tiles), which is what each
// round fetches (1-3 % faster at M = 4608 and 16896, N = 12288).
using TileWide128 = Tile<384, 192, 4, 3, 32, 8, 2, 128>;
// 384 x 96 (each wave 96 x 32): the last, at most half-full round of 384 x 192
// tiles runs as these half-height tiles instead, so it takes about half a
// round (M = 4608, N = 9216: 504 tiles in two rounds, then 144 half tiles;
// 163 us instead of 171 with 256 x 256 tiles over three rounds).
using TileWideHalf = Tile<384, 96, 4, 3, 32, 4, 2, 128>;
// 192 channels x 288 tokens, 12 waves (each 96 x 48 with 16x16x64 MFMAs,
// three waves per SIMD), 128-byte slabs in two stages.  M = 4608 splits into
// 16 token tiles of 288: N = 3072 gives 256 tiles, one full round, where the
// 192 tiles of 384 x 192 leave a quarter of the CUs idle; N = 9216 gives 768,
// three full rounds of three-quarter-size tiles, where 384 x 192 takes two
// rounds and a half-height tail.  Each wave reads a third more LDS bytes per
// MFMA than with 96 x 64 blocks of 32x32 tiles, but its epilogue hides better
// behind the next tile's first MFMAs (18 per wave instead of 6).
using TileTall = Tile<192, 288, 2, 6, 16, 4, 2, 128>;
// A few dozen tokens (16 < M <= 128), where streaming the weight is still most
// of the cost.  With many output channels (N/64 >= 96), 64 channels per
// workgroup and the whole batch in one token tile, so each weight row leaves
// HBM once: 64 x 64 (four waves of 32 x 32) for M <= 64 and 64 x 128 (four
// waves of 32 x 64) for M <= 128, eight 64-byte stages, two workgroups per CU
// (weight from HBM, K = 4096, N = 12288: M = 64 in 16.4 us instead of 28.2
// with 128 x 128 tiles, M = 128 in 20.9 instead of 29.0).  With fewer
// channels, narrower tiles give more workgroups: 32 x 32 (TileSkinny) up to
// M = 64 and 64 x 32 (two waves of 32 x 32, twelve stages) up to M = 128
// (K = 12288, N = 3072: M = 64 in 24.3 us instead of 72.5, M = 128 in 30.6
// instead of 74.7).
using TileM64 = Tile<64, 64, 2, 2, 32, 1, 8>;
using TileM128 = Tile<64, 128, 2, 2, 32, 1, 8>;
using TileM32 = Tile<64, 32, 2, 1, 32, 1, 12>;

typedef int v16i __attribute__((ext_vector_type(16)));

// LDS chunk swizzle of row r (rows are 64 bytes = four 16-byte chunks; chunk c
// of row r is stored at c ^ swz(r)).  On gfx950 a ds_read_b128 is served per
// half-wave (lanes 0-31, then 32-63) in two 256-byte passes: it runs without
// bank conflicts when, within each half, every 16-byte slot of a 256-byte
// window is hit by exactly two lanes (fitted to SQ_LDS_BANK_CONFLICT
// measurements of fifteen access patterns).  A 16x16x64 fragment half reads
// rows 0-15 at chunks c and c+1; a 32x32x32 fragment half reads rows 0-31 at
// one chunk.  Row r sits at slot (r & 3) * 4 + stored chunk, so:
//   16x16: (r >> 1) & 3 spreads rows {q, q+4, q+8, q+12} x 2 chunks evenly;
//   32x32: (r >> 2) & 3 spreads rows {q, q+4, ..., q+28} over 4 chunks twice.
// With 128-byte rows (eight chunks) row r sits at slot (r & 1) * 8 + stored
// chunk, and (r >> 1) & 7 gives each of the 16 slots exactly two of the 32
// rows of a 32x32 half (or of the 16 rows x 2 chunks of a 16x16 half).
template <int MF, int BK>
__device__ inline int swz(int r) {
  if constexpr (BK == 128) return (r >> 1) & 7;
  else if constexpr (MF == 16) return (r >> 1) & 3;
  else return (r >> 2) & 3;
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Operand kinds: int8 codes (int32 accumulator) or the default path's bf16 /
// fp16 values (fp32 accumulator).  Each lane supplies 16 bytes per MFMA.
enum Op { kOpI8 = 0, kOpBf16 = 1, kOpF16 = 2 };

template <int MF, int OP> struct Acc;
template <> struct Acc<16, kOpI8> { using type = v4i; };
template <> struct Acc<32, kOpI8> { using type = v16i; };
template <int OP> struct Acc<16, OP> { using type = v4f; };
template <int OP> struct Acc<32, OP> { using type = v16f; };

template <int MF, int OP>
__device__ inline typename Acc<MF, OP>::type mfma(v4i a, v4i b, typename Acc<MF, OP>::type c) {
  if constexpr (OP == kOpI8) {
    if constexpr (MF == 16) return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  } else if constexpr (OP == kOpBf16) {
    const v8bf a8 = __builtin_bit_cast(v8bf, a), b8 = __builtin_bit_cast(v8bf, b);
    if constexpr (MF == 16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, c, 0, 0, 0);
  } else {
    const v8h a8 = __builtin_bit_cast(v8h, a), b8 = __builtin_bit_cast(v8h, b);
    if constexpr (MF == 16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, b8, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, b8, c, 0, 0, 0);
  }
}

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

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even and packed, a in the low half: one
// v_cvt_pk_bf16_f32 with both sources (converting the two values one by one
// takes two conversions, a shift and an or).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{a, b}), v2bf));
}


// Byte offset of element (row m, column n) of the bf16 output tile staged in
// LDS: rows of BN*2 bytes, 16-byte chunks XOR-swizzled by the low bits of the
// row (as many bits, up to 4, as divide the row's chunk count, so the XOR
// stays inside the row).
template <class T>
__device__ inline int out_lds_offset(int m, int n) {
  constexpr int kChunks = T::BN / 8;
  constexpr int kMask = kChunks % 16 == 0 ? 15 : kChunks % 8 == 0 ? 7 : kChunks % 4 == 0 ? 3 : kChunks - 1;
  static_assert(kChunks % (kMask + 1) == 0 && (kMask & (kMask + 1)) == 0, "chunk swizzle group");
  return m * (T::BN * 2) + (((n >> 3) ^ (m & kMask)) << 4) + ((n & 7) << 1);
}

// Epilogue modes: raw int32 products, or dequant + bias to bf16 / fp16 with
// one weight scale (tensorwise) or one per output channel (row-wise); or the
// default path's bf16 / fp16 product with the bias added (no scales).
enum Epi { kEpiI32 = 0, kEpiBf16 = 1, kEpiBf16Row = 2, kEpiF16 = 3, kEpiF16Row = 4,
           kEpiDefBf16 = 5, kEpiDefF16 = 6 };

// The same for IEEE binary16 (v_cvt_pk_f16_f32, round to nearest even).
__device__ inline uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{a, b}), v2h));
}
__device__ inline float f16_bits_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ inline float f16_bits_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

template <class T, int EPI>
__global__ __launch_bounds__(T::kThreads) void gemm_i8_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    int tiles_n, int tiles_m, const float* __restrict__ x_scale,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
  constexpr bool DEQUANT = EPI != kEpiI32;
  constexpr bool kRowScale = EPI == kEpiBf16Row || EPI == kEpiF16Row;
  constexpr bool kDefault = EPI == kEpiDefBf16 || EPI == kEpiDefF16;
  constexpr bool kF16 = EPI == kEpiF16 || EPI == kEpiF16Row || EPI == kEpiDefF16;
  constexpr int OP = EPI == kEpiDefBf16 ? kOpBf16 : EPI == kEpiDefF16 ? kOpF16 : kOpI8;

  int tn, tm;
  tile_coords<T>(tiles_n, tiles_m, tn, tm);
  const int n0 = tn * T::BN, m0 = tm * T::BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave: keep it in a scalar register,
  // so that LDS destinations (M0) are computed by the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / T::WM, wm = wave % T::WM;

  // ---- direct-to-LDS sources: instruction j of this wave fills LDS rows
  // [16*i, 16*i + 16) of its operand (i = wave * loads + j); lane L lands in
  // row 16*i + L/4, stored chunk L%4, and so fetches global chunk
  // (L%4) ^ ((row >> 1) & 3) of that row.
  // Each load's global address is a per-tile scalar base (the tile's first
  // row of the operand, plus the slab's K offset) and a per-lane 32-bit
  // offset that stays fixed for the whole K loop (at most BN rows of K bytes,
  // far below 2^31), so no vector instruction recomputes an address between
  // the loads of a slab.
  const int8_t* a_tile = wq + static_cast<int64_t>(n0) * K;
  const int8_t* b_tile = xq + static_cast<int64_t>(m0) * K;
  uint32_t off[T::kLoads];
  int dst[T::kLoads];
#pragma unroll
  for (int j = 0; j < T::kLoads; ++j) {
    const bool is_a = j < T::kALoads;
    const int i = is_a ? wave * T::kALoads + j : wave * T::kBLoads + (j - T::kALoads);
    const int row = T::kRowsPerLoad * i + lane / T::kRowChunks;
    const int chunk = (lane % T::kRowChunks) ^ swz<T::MF, T::BK>(row);
    if (is_a) {
      off[j] = static_cast<uint32_t>((min(n0 + row, N - 1) - n0) * K + chunk * 16);
      dst[j] = i * T::kRowsPerLoad * T::BK;
    } else {
      off[j] = static_cast<uint32_t>((min(m0 + row, M - 1) - m0) * K + chunk * 16);
      dst[j] = T::BN * T::BK + i * T::kRowsPerLoad * T::BK;
    }
  }
  const int KT = K / T::BK;

  auto issue_slab = [&](int slab, int stage) {
    const int64_t k0 = static_cast<int64_t>(slab) * T::BK;
#pragma unroll
    for (int j = 0; j < T::kLoads; ++j) {
      const int8_t* base = (j < T::kALoads ? a_tile : b_tile) + k0;
      // keep the offset a 32-bit register at the load (the empty asm makes it
      // opaque, so the compiler cannot widen it ahead of the loop and the load
      // takes the scalar base + 32-bit vector offset form)
      asm volatile("" : "+v"(off[j]));
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[j]),
                                       (lds_void_t*)(lds + stage * T::kStageBytes + dst[j]),
                                       16, 0, 0);
    }
  };

  // ---- fragment reads.  16x16x64: lane reads row (l & 15) of a 16-row block,
  // chunk l >> 4.  32x32x32: row (l & 31) of a 32-row block, chunk
  // 2 * kstep + (l >> 5).  Stored chunk = chunk ^ swz(row).
  constexpr int kRowMask = T::MF - 1;
  constexpr int kChunkShift = T::MF == 16 ? 4 : 5;
  const int frow = lane & kRowMask;
  int frag[T::kKSteps];
#pragma unroll
  for (int kk = 0; kk < T::kKSteps; ++kk) {
    const int chunk = kk * (T::kUnitBytes / 16) + (lane >> kChunkShift);
    frag[kk] = frow * T::BK + (((chunk ^ swz<T::MF, T::BK>(frow)) & (T::kRowChunks - 1)) << 4);
  }
  const int a_base = wn * T::kWaveN * T::BK;
  const int b_base = T::BN * T::BK + wm * T::kWaveM * T::BK;

  using acc_t = typename Acc<T::MF, OP>::type;
  acc_t acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = acc_t{};

  // Token scales of this lane's output columns, fetched before the main loop
  // so that their latency hides behind it (the dequant epilogue only).
  float alpha[T::TM];
  const int m_lane0 = wm * T::kWaveM + (lane & (T::MF - 1));
#pragma unroll
  for (int j = 0; j < T::TM; ++j)
    alpha[j] = DEQUANT && !kDefault ? x_scale[min(m0 + m_lane0 + j * T::MF, M - 1)] : 0.0f;
  (void)w_scale;

  // Fragments are double-buffered per MFMA k step (a "unit": 32 bytes of K
  // for 32x32x32, 64 for 16x16x64): while the MFMAs of one unit run from one
  // register set, the LDS reads of the next unit fill the other.  Only two
  // units' fragments are ever live, which keeps the 12-wave tile within its
  // 168 registers.  The unit after the last of slab kt is the first of slab
  // kt+1, which the barrier at the top of step kt has made visible.
  struct KFrag { v4i a[T::TN], b[T::TM]; };
  auto read_unit = [&](int slab_stage, int kk, KFrag& f) {
    const char* st = lds + slab_stage * T::kStageBytes;
#pragma unroll
    for (int t = 0; t < T::TM; ++t)
      f.b[t] = *reinterpret_cast<const v4i*>(st + b_base + t * T::MF * T::BK + frag[kk]);
#pragma unroll
    for (int t = 0; t < T::TN; ++t)
      f.a[t] = *reinterpret_cast<const v4i*>(st + a_base + t * T::MF * T::BK + frag[kk]);
  };
  auto compute_unit = [&](const KFrag& f) {
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
      for (int j = 0; j < T::TM; ++j) acc[i][j] = mfma<T::MF, OP>(f.a[i], f.b[j], acc[i][j]);
  };
  // Issue order inside a unit: each MFMA is followed by one of the unit's
  // loads (direct-to-LDS loads first, then LDS fragment reads), so the loads
  // issue while the matrix unit works instead of in a burst before it.
  constexpr int kUnitMfmas = T::TN * T::TM;
  constexpr int kUnitReads = T::TN + T::TM;
  auto order_unit = [&](auto loads_c) {
    constexpr int kV = decltype(loads_c)::value;
    constexpr int kPairV = kV < kUnitMfmas ? kV : kUnitMfmas;
    constexpr int kPairD = kUnitReads < kUnitMfmas - kPairV ? kUnitReads : kUnitMfmas - kPairV;
#pragma unroll
    for (int i = 0; i < kPairV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM (direct-to-LDS load)
    }
#pragma unroll
    for (int i = 0; i < kPairD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    }
    if constexpr (kUnitMfmas > kPairV + kPairD)
      __builtin_amdgcn_sched_group_barrier(0x008, kUnitMfmas - kPairV - kPairD, 0);
    if constexpr (kV > kPairV) __builtin_amdgcn_sched_group_barrier(0x010, kV - kPairV, 0);
    if constexpr (kUnitReads > kPairD)
      __builtin_amdgcn_sched_group_barrier(0x100, kUnitReads - kPairD, 0);
    __builtin_amdgcn_sched_barrier(0);   // nothing crosses into the next unit
  };
  // Slab-boundary unit of the two-stage pipeline: its MFMAs carry all of the
  // next slab's direct-to-LDS loads and the next unit's fragment reads, one
  // of each after every MFMA.
  auto order_boundary = [&]() {
    constexpr int kV = T::kLoads;
    constexpr int kT = kV < kUnitReads ? (kV < kUnitMfmas ? kV : kUnitMfmas)
                                       : (kUnitReads < kUnitMfmas ? kUnitReads : kUnitMfmas);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM (direct-to-LDS load)
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    }
    if constexpr (kUnitMfmas > kT) __builtin_amdgcn_sched_group_barrier(0x008, kUnitMfmas - kT, 0);
    if constexpr (kV > kT) __builtin_amdgcn_sched_group_barrier(0x010, kV - kT, 0);
    if constexpr (kUnitReads > kT) __builtin_amdgcn_sched_group_barrier(0x100, kUnitReads - kT, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // One pipeline step on slab kt (x holds its first unit on entry; on exit
  // the register set named by the return value holds slab kt+1's first
  // unit): wait until slab kt+1 has landed (only slab kt+2 may still be in
  // flight) and everyone is done reading the stage of slab kt-1, refill that
  // stage with slab kt+3, then run the slab's units.  Slab indices past the
  // end re-fetch the last slab into stages that are never read for results.
  auto step = [&](int kt, KFrag& x, KFrag& y) {
    wait_vm_barrier<(T::kStages >= 3 ? (T::kStages - 3) * T::kLoads : 0)>();
    issue_slab(min(kt + T::kStages - 1, KT - 1), (kt + T::kStages - 1) % T::kStages);
    if constexpr (T::kKSteps == 2) {
      read_unit(kt % T::kStages, 1, y);
      compute_unit(x);
      order_unit(std::integral_constant<int, T::kLoads>{});
      read_unit((kt + 1) % T::kStages, 0, x);
      compute_unit(y);
      order_unit(std::integral_constant<int, 0>{});
    } else {
      read_unit((kt + 1) % T::kStages, 0, y);
      compute_unit(x);
      order_unit(std::integral_constant<int, T::kLoads>{});
    }
  };

  if constexpr (T::kStages > 2) {
#pragma unroll
    for (int s = 0; s < T::kStages - 1; ++s) issue_slab(min(s, KT - 1), s);
  }
  KFrag f0, f1;
  if constexpr (T::kStages == 2) {
    // Two stages: slab kt+2 is issued at the boundary between slabs kt and
    // kt+1, into the stage slab kt occupied; by then slab kt+1 has landed and
    // every wave holds slab kt's last unit in registers.  Units alternate
    // between the register sets (an even count per slab, so every slab starts
    // in f0).
    static_assert(T::kKSteps % 2 == 0, "even unit count per slab");
    issue_slab(0, 0);
    issue_slab(min(1, KT - 1), 1);
    wait_vm_barrier<T::kLoads>();      // slab 0 has landed, slab 1 may be in flight
    read_unit(0, 0, f0);
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt & 1;
#pragma unroll
      for (int u = 0; u + 2 < T::kKSteps; u += 2) {
        read_unit(st, u + 1, f1);
        compute_unit(f0);
        order_unit(std::integral_constant<int, 0>{});
        read_unit(st, u + 2, f0);
        compute_unit(f1);
        order_unit(std::integral_constant<int, 0>{});
      }
      read_unit(st, T::kKSteps - 1, f1);
      compute_unit(f0);
      order_unit(std::integral_constant<int, 0>{});
      // slab boundary (slab indices past the end re-fetch the last slab into
      // a stage that is never read for results)
      wait_vm_barrier<0>();
      issue_slab(min(kt + 2, KT - 1), st);
      read_unit(st ^ 1, 0, f0);
      compute_unit(f1);
      order_boundary();
    }
  } else {
    static_assert(T::kKSteps <= 2, "three-plus stage pipeline runs one or two units per slab");
    wait_vm_barrier<(T::kStages - 2) * T::kLoads>();
    read_unit(0, 0, f0);
    // The loop runs in slab pairs with fixed register roles.  One unit per
    // slab (64-byte slabs): K is a multiple of 128, so KT is even.  Two units
    // per slab: every step leaves the next slab's first unit in f0, so an
    // odd KT (128-byte slabs) just skips the last pair's second step.
    for (int kt = 0; kt < KT; kt += 2) {
      if constexpr (T::kKSteps == 2) {
        step(kt, f0, f1);       // f0 <- first unit of slab kt+1
        if (kt + 1 < KT) step(kt + 1, f0, f1);
      } else {
        step(kt, f0, f1);       // f1 <- slab kt+1
        step(kt + 1, f1, f0);
      }
    }
  }

  // Lane layout of a result block (rows n = weight rows, columns m = tokens):
  //   16x16: acc[i][j][e]        -> n = i*16 + 4*(l >> 4) + e,           m = j*16 + (l & 15)
  //   32x32: acc[i][j][4*g + e]  -> n = i*32 + 8*g + 4*(l >> 5) + e,     m = j*32 + (l & 31)
  // (n and m relative to this wave's corner; e = 0..3 are consecutive n).
  constexpr int kGroups = T::kAccRegs / 4;
  const int n_loc = wn * T::kWaveN + 4 * (lane >> kChunkShift);
  const int m_loc = wm * T::kWaveM + (lane & kRowMask);

  if constexpr (DEQUANT) {
    uint16_t* y = static_cast<uint16_t*>(out);
    // Scales and bias for this lane's outputs: every load is issued before
    // the first one is used, so their latency is paid once per tile.
    const float sw = kRowScale || kDefault ? 1.0f : *w_scale;
    // bias of n = n0 + n_loc + i*MF + 8*g + e, e = 0..3: 8-byte loads when the
    // four values are in range and aligned, else element by element
    uint2 bias4[T::TN][kGroups];
    // row-wise weight scales of the same four channels, loaded one MFMA row
    // block (i) at a time below: all of them at once would not fit beside
    // the accumulators
    const bool ws_vec = kRowScale && (N & 3) == 0 && (reinterpret_cast<uintptr_t>(w_scale) & 15) == 0;
    auto load_ws = [&](int i, int g) -> float4 {
      const int n = n0 + n_loc + i * T::MF + 8 * g;
      if (ws_vec) return *reinterpret_cast<const float4*>(w_scale + min(n, N - 4));
      return make_float4(w_scale[min(n, N - 1)], w_scale[min(n + 1, N - 1)],
                         w_scale[min(n + 2, N - 1)], w_scale[min(n + 3, N - 1)]);
    };
    const bool bias_vec = bias != nullptr && (N & 3) == 0 && (reinterpret_cast<uintptr_t>(bias) & 7) == 0;
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int n = n0 + n_loc + i * T::MF + 8 * g;
        if (bias_vec) {
          bias4[i][g] = *reinterpret_cast<const uint2*>(bias + min(n, N - 4));
        } else if (bias != nullptr) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = bias[min(n + e, N - 1)];
          bias4[i][g] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
          bias4[i][g] = make_uint2(0u, 0u);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < T::TM; ++j) alpha[j] = alpha[j] * sw;
    // every wave is done with the stages (and every load has landed) before
    // the output tile overwrites them
    wait_vm_barrier<0>();
#pragma unroll
    for (int i = 0; i < T::TN; ++i) {
      float4 ws4[kRowScale ? kGroups : 1];
      if constexpr (kRowScale) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) ws4[g] = load_ws(i, g);
      }
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int nl = n_loc + i * T::MF + 8 * g;
        float b[4];
        if constexpr (kF16) {
          b[0] = f16_bits_lo(bias4[i][g].x); b[1] = f16_bits_hi(bias4[i][g].x);
          b[2] = f16_bits_lo(bias4[i][g].y); b[3] = f16_bits_hi(bias4[i][g].y);
        } else {
          b[0] = __uint_as_float(bias4[i][g].x << 16); b[1] = __uint_as_float(bias4[i][g].x & 0xffff0000u);
          b[2] = __uint_as_float(bias4[i][g].y << 16); b[3] = __uint_as_float(bias4[i][g].y & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < T::TM; ++j) {
          float v[4];
          if constexpr (kDefault) {
            // default path: fp32 product sum plus the bias, one rounding below
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + b[e];
          } else if constexpr (kRowScale) {
            // alpha = s_x[m] * s_w[n], one fp32 product per output
            const float sc[4] = {ws4[g].x, ws4[g].y, ws4[g].z, ws4[g].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = __builtin_fmaf(static_cast<float>(acc[i][j][4 * g + e]), alpha[j] * sc[e], b[e]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = __builtin_fmaf(static_cast<float>(acc[i][j][4 * g + e]), alpha[j], b[e]);
          }
          if constexpr (kF16) {
            // the output is fp16_rne of the fp32 result: keep v in fp32 here,
            // or the compiler fuses the fma (or add) and the conversion into
            // v_fma_mixlo_f16, which rounds the exact value to fp16 once
#pragma unroll
            for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(v[e]));
          }
          *reinterpret_cast<uint2*>(lds + out_lds_offset<T>(m_loc + j * T::MF, nl)) =
              kF16 ? make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]))
                   : make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
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
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int n = n0 + n_loc + i * T::MF + 8 * g;
#pragma unroll
        for (int j = 0; j < T::TM; ++j) {
          const int m = m0 + m_loc + j * T::MF;
          if (m >= M) continue;
          int32_t* dstp = c + static_cast<int64_t>(m) * N + n;
          const int a0 = acc[i][j][4 * g], a1 = acc[i][j][4 * g + 1];
          const int a2 = acc[i][j][4 * g + 2], a3 = acc[i][j][4 * g + 3];
          if (vec && n + 3 < N) {
            *reinterpret_cast<int4*>(dstp) = make_int4(a0, a1, a2, a3);
          } else {
            if (n < N) dstp[0] = a0;
            if (n + 1 < N) dstp[1] = a1;
            if (n + 2 < N) dstp[2] = a2;
            if (n + 3 < N) dstp[3] = a3;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- few tokens, K split over waves

// The end of a K-split few-token tile: waves 1-3 park their 16 x 16 partial
// sums in LDS, wave 0 adds them (integer sums: the result does not depend on
// the split) and runs the epilogue.  Lane l holds channels n0 + 4 (l >> 4) + e
// of token l & 15.
template <int EPI, typename AccT>
__device__ inline void ksplit_finish(AccT acc, v4i (&red)[3][64], int wave, int lane, int n0, int M, int N,
                                     const float* __restrict__ x_scale, const float* __restrict__ w_scale,
                                     const uint16_t* __restrict__ bias, void* __restrict__ out) {
  constexpr bool DEQUANT = EPI != kEpiI32;
  constexpr bool kRowScale = EPI == kEpiBf16Row || EPI == kEpiF16Row;
  constexpr bool kDefault = EPI == kEpiDefBf16 || EPI == kEpiDefF16;
  constexpr bool kF16 = EPI == kEpiF16 || EPI == kEpiF16Row || EPI == kEpiDefF16;
  constexpr int OP = EPI == kEpiDefBf16 ? kOpBf16 : EPI == kEpiDefF16 ? kOpF16 : kOpI8;
  if (wave > 0) red[wave - 1][lane] = __builtin_bit_cast(v4i, acc);
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const v4i p = red[w][lane];
    if constexpr (OP == kOpI8) acc += p;
    else acc += __builtin_bit_cast(v4f, p);
  }
  const int m = lane & 15;
  const int n = n0 + 4 * (lane >> 4);
  if (m >= M) return;
  if constexpr (!DEQUANT) {
    int32_t* c = static_cast<int32_t*>(out) + static_cast<int64_t>(m) * N + n;
    if ((N & 3) == 0 && n + 3 < N) {
      *reinterpret_cast<int4*>(c) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) c[e] = acc[e];
    }
  } else {
    float alpha = 0.0f;
    if constexpr (!kDefault) alpha = kRowScale ? x_scale[m] : x_scale[m] * *w_scale;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ne = min(n + e, N - 1);
      float b = 0.0f;
      if (bias != nullptr)
        b = kF16 ? static_cast<float>(__builtin_bit_cast(_Float16, bias[ne]))
                 : __uint_as_float(static_cast<uint32_t>(bias[ne]) << 16);
      if constexpr (kDefault) v[e] = acc[e] + b;
      else if constexpr (kRowScale) v[e] = __builtin_fmaf(static_cast<float>(acc[e]), alpha * w_scale[ne], b);
      else v[e] = __builtin_fmaf(static_cast<float>(acc[e]), alpha, b);
    }
    uint32_t w0, w1;
    if constexpr (kF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(v[e]));
      w0 = pack_f16x2(v[0], v[1]);
      w1 = pack_f16x2(v[2], v[3]);
    } else {
      w0 = pack_bf16x2(v[0], v[1]);
      w1 = pack_bf16x2(v[2], v[3]);
    }
    uint16_t* y = static_cast<uint16_t*>(out) + static_cast<int64_t>(m) * N + n;
    if ((N & 3) == 0 && n + 3 < N) {
      *reinterpret_cast<uint2*>(y) = make_uint2(w0, w1);
    } else {
      const uint32_t ww[2] = {w0, w1};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n + e < N) y[e] = static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// M <= 16: the weight stream is the whole cost, and a workgroup per 16 output
// channels leaves one wave per workgroup to issue its loads.  Here the four
// waves of a workgroup split K: wave w runs slabs [w KT / 4, (w + 1) KT / 4)
// of 128 bytes (16 weight rows and the 16 token rows, 4 KB, four
// direct-to-LDS loads of eight full 128-byte rows) through its own S-stage
// ring in LDS, so the waves need no barrier until the end.  There waves 1-3
// park their 16 x 16 int32 partial sums in LDS and wave 0 adds them (integer
// sums: the result does not depend on the split) and runs the epilogue.
// The default path's fp32 product takes the same route; its sum order then
// differs from the other tiles' in the last bits, within its tolerance.
// Two stages per wave (32 KB per workgroup, three per CU): weight from HBM,
// 16 x 12288 x 4096 in 11.5 us against 12.2 with the one-wave tile (three
// stages 11.9, four 16.1; loading the operands straight into registers,
// 16 rows x 64 bytes per instruction, 17.4).  With N / 16 below twice the
// CU count the one-wave tile is faster (16 x 3072 x 12288: 13.2 us against
// 18.4): each wave's share of K is then too short.
template <int EPI, int S>
__global__ __launch_bounds__(256) void gemm_ksplit_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  constexpr int OP = EPI == kEpiDefBf16 ? kOpBf16 : EPI == kEpiDefF16 ? kOpF16 : kOpI8;
  constexpr int kStage = 4096;                      // A: 16 rows x 128 B, then B: 16 rows x 128 B
  __shared__ __attribute__((aligned(16))) char lds[4 * S * kStage];
  __shared__ __attribute__((aligned(16))) v4i red[3][64];
  using acc_t = typename Acc<16, OP>::type;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int KT = K / 128;
  const int kt0 = wave * KT / 4, nk = (wave + 1) * KT / 4 - kt0;
  char* wl = lds + wave * S * kStage;
  // a load fills eight 128-byte LDS rows: lane -> row 8 i + (lane >> 3),
  // stored chunk lane & 7, fetched global chunk (lane & 7) ^ swz(row); rows
  // past N or M read the last valid row (results discarded)
  uint32_t off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (j & 1) + (lane >> 3);
    const int c16 = ((lane & 7) ^ swz<16, 128>(row)) * 16;
    off[j] = j < 2 ? static_cast<uint32_t>((min(n0 + row, N - 1) - n0) * K + c16)
                   : static_cast<uint32_t>(min(row, M - 1) * K + c16);
  }
  const int8_t* a_tile = wq + static_cast<int64_t>(n0) * K;
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int8_t* base = (j < 2 ? a_tile : xq) + static_cast<int64_t>(kt) * 128;
      asm volatile("" : "+v"(off[j]));
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[j]),
                                       (lds_void_t*)(wl + stage * kStage + (j >> 1) * 2048 + (j & 1) * 1024),
                                       16, 0, 0);
    }
  };
  // 16x16x64 fragment of unit kk (0, 1) of a slab: row lane & 15, chunk
  // 4 kk + (lane >> 4)
  const int frow = lane & 15;
  int frag[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) frag[kk] = frow * 128 + (((4 * kk + (lane >> 4)) ^ swz<16, 128>(frow)) << 4);

  acc_t acc = acc_t{};
  if (nk > 0) {
    // every step issues exactly one slab (past the end: the wave's last slab
    // again, into the stage just finished, never read), so the wait count
    // is fixed
#pragma unroll
    for (int s2 = 0; s2 < S - 1; ++s2) issue(kt0 + min(s2, nk - 1), s2);
    for (int i = 0; i < nk; ++i) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * 4) : "memory");
      issue(kt0 + min(i + S - 1, nk - 1), (i + S - 1) % S);
      const char* st = wl + (i % S) * kStage;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const v4i a = *reinterpret_cast<const v4i*>(st + frag[kk]);
        const v4i b = *reinterpret_cast<const v4i*>(st + 2048 + frag[kk]);
        acc = mfma<16, OP>(a, b, acc);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  ksplit_finish<EPI>(acc, red, wave, lane, n0, M, N, x_scale, w_scale, bias, out);
}

// The same K split for K = 512 NK (each wave NK slabs: K = 3072 and 4096),
// with the operands streamed through registers: a lane loads 16 bytes of a
// 128-byte row piece (eight lanes per row, eight rows per load, whole cache
// lines), four slabs ahead, and writes each slab into a wave-private
// two-stage LDS ring in the MFMA layout, from which the fragments are read as
// in the kernel above.  A timing probe of the two weight paths alone (768
// workgroups of four waves, 50 MB from HBM) gave 10.1-10.5 us through
// direct-to-LDS rings of any depth and 6.9-7.3 us through registers with four
// to eight slabs in flight.  The steps are unrolled, so the compiler's wait
// counts stay exact (in a rolled loop they fell back to waiting for every
// load at each pass).  16 x 12288 x 4096: 10.7-10.8 us instead of 11.4-11.5;
// 16 x 12288 x 3072: 8.7-8.8 instead of 9.4.
template <int EPI, int NK>
__global__ __launch_bounds__(256) void gemm_ksplit_reg_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    const float* __restrict__ x_scale, const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  constexpr int OP = EPI == kEpiDefBf16 ? kOpBf16 : EPI == kEpiDefF16 ? kOpF16 : kOpI8;
  constexpr int kStage = 4096;                      // A: 16 rows x 128 B, then B: 16 rows x 128 B
  constexpr int kAhead = 4;                         // slabs in flight per wave
  __shared__ __attribute__((aligned(16))) char lds[4 * 2 * kStage];
  __shared__ __attribute__((aligned(16))) v4i red[3][64];
  using acc_t = typename Acc<16, OP>::type;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 16;
  const int kt0 = wave * NK;
  char* wl = lds + wave * 2 * kStage;
  // a slab is four 16-byte loads per lane: j = 0, 1 the weight rows
  // 8 j + (lane >> 3), j = 2, 3 the token rows 8 (j - 2) + (lane >> 3), chunk
  // lane & 7 of the slab's 128 bytes; rows past N or M read the last valid
  // row (results discarded).  In LDS the chunk goes to slot
  // (lane & 7) ^ swz(row), the layout the direct-to-LDS loads above produce.
  uint32_t goff[4];
  int loff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (j & 1) + (lane >> 3);
    const int c16 = (lane & 7) * 16;
    goff[j] = j < 2 ? static_cast<uint32_t>((min(n0 + row, N - 1) - n0) * K + c16)
                    : static_cast<uint32_t>(min(row, M - 1) * K + c16);
    loff[j] = (j >> 1) * 2048 + row * 128 + (((lane & 7) ^ swz<16, 128>(row)) << 4);
  }
  const int8_t* a_tile = wq + static_cast<int64_t>(n0) * K;
  v4i buf[kAhead][4];
  auto load = [&](int kt, v4i (&r)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r[j] = *reinterpret_cast<const v4i*>((j < 2 ? a_tile : xq) + static_cast<int64_t>(kt) * 128 + goff[j]);
  };
  const int frow = lane & 15;
  int frag[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) frag[kk] = frow * 128 + (((4 * kk + (lane >> 4)) ^ swz<16, 128>(frow)) << 4);

  acc_t acc = acc_t{};
#pragma unroll
  for (int d = 0; d < kAhead && d < NK; ++d) load(kt0 + d, buf[d]);
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    char* st = wl + (i & 1) * kStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<v4i*>(st + loff[j]) = buf[i % kAhead][j];
    if (i + kAhead < NK) load(kt0 + i + kAhead, buf[i % kAhead]);
    // the wave reads what its own lanes just wrote (and wrote over what it
    // read two slabs ago): a wave's LDS accesses complete in order
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const v4i a = *reinterpret_cast<const v4i*>(st + frag[kk]);
      const v4i b = *reinterpret_cast<const v4i*>(st + 2048 + frag[kk]);
      acc = mfma<16, OP>(a, b, acc);
    }
  }
  ksplit_finish<EPI>(acc, red, wave, lane, n0, M, N, x_scale, w_scale, bias, out);
}

// ---------------------------------------------------------------- persistent two-stage tiles
//
// One workgroup per CU walks its share of the tiles (the same XCD-aware order
// as the one-tile-per-workgroup kernel) and keeps the operand pipeline running
// across tile boundaries: the slab after next is issued at every slab
// boundary, also when it belongs to the next tile, so a new tile finds its
// first slab landed and its second in flight.  The epilogue needs no LDS and
// no barrier: each wave converts its accumulators, exchanges halves between
// lanes 32 apart (v_permlane32_swap) so that every lane holds eight
// consecutive output channels of one token, and stores them as 16-byte
// pieces; the wave then goes straight on to the next tile's first slab while
// the stores drain, and the next slab boundary waits only for the loads
// issued before those stores (vector memory counts complete in issue order).
// When the tile is whole and another follows, the next tile's first MFMA
// unit runs inside the epilogue: each result block, once converted and
// stored, restarts with that unit's MFMA, so the matrix cores are not idle
// while the epilogue's vector work runs.
// Token scales, weight scales and bias of a tile are fetched into registers
// when the tile starts (one or two values per thread) and parked in a
// double-buffered LDS table at its last slab boundary.  Three or more slabs
// per tile (K >= 384).  With 16x16 result blocks a lane holds four channels
// of one token; v_permlane16_swap between the blocks of two neighbouring
// channel tiles gives every lane eight consecutive channels.
template <class T, int EPI>
__global__ __launch_bounds__(T::kThreads) void gemm_persist_kernel(
    const int8_t* __restrict__ wq, const int8_t* __restrict__ xq, int M, int N, int K,
    int tiles_n, int tiles_m, const float* __restrict__ x_scale,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ bias,
    void* __restrict__ out) {
  static_assert(T::kStages == 2 && T::BK == 128 && T::kKSteps % 2 == 0, "two 128-byte stages");
  static_assert(T::MF == 32 || T::TN % 2 == 0, "16x16 result blocks are stored in pairs along n");
  constexpr bool DEQUANT = EPI != kEpiI32;
  constexpr bool kRowScale = EPI == kEpiBf16Row || EPI == kEpiF16Row;
  constexpr bool kDefault = EPI == kEpiDefBf16 || EPI == kEpiDefF16;
  constexpr bool kF16 = EPI == kEpiF16 || EPI == kEpiF16Row || EPI == kEpiDefF16;
  constexpr int OP = EPI == kEpiDefBf16 ? kOpBf16 : EPI == kEpiDefF16 ? kOpF16 : kOpI8;
  // parameter table: bias [BN], row scales [BN] (row mode), token factors [BM]
  constexpr int kPBias = 0;
  constexpr int kPWs = T::BN;
  constexpr int kPAlpha = kRowScale ? 2 * T::BN : T::BN;
  constexpr int kParams = DEQUANT ? kPAlpha + (kDefault ? 0 : T::BM) : 0;
  constexpr int kParamPerThread = (kParams + T::kThreads - 1) / T::kThreads;
  // 16-byte output pieces per lane and tile (interior tiles): two per 32 x 32
  // block, one per pair of 16 x 16 blocks
  constexpr int kStores = T::MF == 32 ? T::TN * T::TM * 2 : T::TN * T::TM / 2;
  constexpr int kParamFloats = ((kParams > 0 ? kParams : 1) + 3) / 4 * 4;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes + 2 * kParamFloats * 4];
  float* ptab0 = reinterpret_cast<float*>(lds + T::kLdsBytes);

  const int total = tiles_n * tiles_m;
  // this workgroup's tiles: its XCD's contiguous run of the tile order,
  // every wgs-th one (wgs = workgroups on this XCD)
  const int nb = gridDim.x;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int wgs = (nb >> 3) + (xcd < (nb & 7) ? 1 : 0);
  const int run_len = total / 8 + (xcd < total % 8 ? 1 : 0);
  const int run0 = xcd * (total / 8) + min(xcd, total % 8);
  auto tile_of = [&](int i, int& tn, int& tm) -> bool {   // i-th tile of this workgroup
    const int r = local + i * wgs;
    if (r >= run_len) return false;
    const int v = run0 + r;
    const int per_group = T::kGroupM * tiles_n;
    const int gid = v / per_group;
    const int first_m = gid * T::kGroupM;
    const int gsz = min(tiles_m - first_m, T::kGroupM);
    const int in_group = v - gid * per_group;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
    return true;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / T::WM, wm = wave % T::WM;
  const int KT = K / T::BK;

  // ---- load cursor: the tile whose slabs are being issued (base pointers
  // and the byte offset of its last valid row in each operand, for clamping
  // ragged edges) and the next slab index.  A row past the edge is read as
  // the same chunk of the last valid row.
  struct Cursor { const int8_t* a; const int8_t* b; uint32_t last_a, last_b; };
  auto cursor_of = [&](int tn, int tm) {
    const int n0 = tn * T::BN, m0 = tm * T::BM;
    Cursor c;
    c.a = wq + static_cast<int64_t>(n0) * K;
    c.b = xq + static_cast<int64_t>(m0) * K;
    c.last_a = static_cast<uint32_t>((min(N - n0, T::BN) - 1) * K);
    c.last_b = static_cast<uint32_t>((min(M - m0, T::BM) - 1) * K);
    return c;
  };
  // per-lane offsets of the cursor's tile, recomputed when the cursor moves
  // to another tile (from an opaque copy of the lane id, so that nothing of
  // it stays live through the main loop)
  uint32_t off[T::kLoads];
  auto aim = [&](const Cursor& c) {
    int lane_a = lane;
    asm volatile("" : "+v"(lane_a));
#pragma unroll
    for (int j = 0; j < T::kLoads; ++j) {
      const bool is_a = j < T::kALoads;
      const int i = is_a ? wave * T::kALoads + j : wave * T::kBLoads + (j - T::kALoads);
      const int row = T::kRowsPerLoad * i + lane_a / T::kRowChunks;
      const uint32_t c16 = static_cast<uint32_t>(((lane_a % T::kRowChunks) ^ swz<T::MF, T::BK>(row)) * 16);
      off[j] = min(static_cast<uint32_t>(row * K) + c16, (is_a ? c.last_a : c.last_b) + c16);
    }
  };
  Cursor cur_ld;
  int ld_kt = 0;
  // issue slab ld_kt of the cursor's tile into stage `stage` (no branches, so
  // the loads stay in the scheduling region of the MFMAs they are interleaved
  // with)
  auto issue_loads = [&](int stage, auto jb_c, auto je_c) {   // loads [jb, je) of the slab
    const int64_t k0 = static_cast<int64_t>(ld_kt) * T::BK;
#pragma unroll
    for (int j = decltype(jb_c)::value; j < decltype(je_c)::value; ++j) {
      const bool is_a = j < T::kALoads;
      const int i = is_a ? wave * T::kALoads + j : wave * T::kBLoads + (j - T::kALoads);
      const int dst = stage * T::kStageBytes + (is_a ? 0 : T::BN * T::BK) + i * T::kRowsPerLoad * T::BK;
      const int8_t* base = (is_a ? cur_ld.a : cur_ld.b) + k0;
      asm volatile("" : "+v"(off[j]));
      __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[j]), (lds_void_t*)(lds + dst), 16, 0, 0);
    }
  };
  using JA_ = std::integral_constant<int, 0>;
  using JE_ = std::integral_constant<int, T::kLoads>;

  // ---- fragment reads (as in the one-tile kernel)
  constexpr int kRowMask = T::MF - 1;
  constexpr int kChunkShift = T::MF == 16 ? 4 : 5;
  const int frow = lane & kRowMask;
  int frag[T::kKSteps];
#pragma unroll
  for (int kk = 0; kk < T::kKSteps; ++kk) {
    const int chunk = kk * (T::kUnitBytes / 16) + (lane >> kChunkShift);
    frag[kk] = frow * T::BK + (((chunk ^ swz<T::MF, T::BK>(frow)) & (T::kRowChunks - 1)) << 4);
  }
  const int a_base = wn * T::kWaveN * T::BK;
  const int b_base = T::BN * T::BK + wm * T::kWaveM * T::BK;
  using acc_t = typename Acc<T::MF, OP>::type;
  acc_t acc[T::TN][T::TM];
  struct KFrag { v4i a[T::TN], b[T::TM]; };
  auto read_unit = [&](int slab_stage, int kk, KFrag& f) {
    const char* st = lds + slab_stage * T::kStageBytes;
#pragma unroll
    for (int t = 0; t < T::TM; ++t)
      f.b[t] = *reinterpret_cast<const v4i*>(st + b_base + t * T::MF * T::BK + frag[kk]);
#pragma unroll
    for (int t = 0; t < T::TN; ++t)
      f.a[t] = *reinterpret_cast<const v4i*>(st + a_base + t * T::MF * T::BK + frag[kk]);
  };
  auto compute_unit = [&](const KFrag& f) {
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
      for (int j = 0; j < T::TM; ++j) acc[i][j] = mfma<T::MF, OP>(f.a[i], f.b[j], acc[i][j]);
  };
  constexpr int kUnitMfmas = T::TN * T::TM;
  constexpr int kUnitReads = T::TN + T::TM;
  auto order_unit = [&](auto loads_c) {   // MFMAs interleaved with this unit's loads, then its reads
    constexpr int kV = decltype(loads_c)::value;
    constexpr int kPairV = kV < kUnitMfmas ? kV : kUnitMfmas;
    constexpr int kPairD = kUnitReads < kUnitMfmas - kPairV ? kUnitReads : kUnitMfmas - kPairV;
#pragma unroll
    for (int i = 0; i < kPairV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM (direct-to-LDS load)
    }
#pragma unroll
    for (int i = 0; i < kPairD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    }
    if constexpr (kUnitMfmas > kPairV + kPairD)
      __builtin_amdgcn_sched_group_barrier(0x008, kUnitMfmas - kPairV - kPairD, 0);
    if constexpr (kV > kPairV) __builtin_amdgcn_sched_group_barrier(0x010, kV - kPairV, 0);
    if constexpr (kUnitReads > kPairD) __builtin_amdgcn_sched_group_barrier(0x100, kUnitReads - kPairD, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto order_boundary = [&](auto reads_c) {
    constexpr int kV = T::kLoads;
    constexpr int kR = decltype(reads_c)::value ? kUnitReads : 0;
    constexpr int kT = kR == 0 ? (kV < kUnitMfmas ? kV : kUnitMfmas)
                     : kV < kR ? (kV < kUnitMfmas ? kV : kUnitMfmas) : (kR < kUnitMfmas ? kR : kUnitMfmas);
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM (direct-to-LDS load)
      if constexpr (kR > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    }
    if constexpr (kUnitMfmas > kT) __builtin_amdgcn_sched_group_barrier(0x008, kUnitMfmas - kT, 0);
    if constexpr (kV > kT) __builtin_amdgcn_sched_group_barrier(0x010, kV - kT, 0);
    if constexpr (kR > kT) __builtin_amdgcn_sched_group_barrier(0x100, kR - kT, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- a tile's epilogue parameters, one or two per thread, fetched when the
  // tile starts and parked in the LDS table at its epilogue
  float pv[kParamPerThread > 0 ? kParamPerThread : 1];
  auto fetch_params = [&](int n0, int m0) {
#pragma unroll
    for (int r = 0; r < kParamPerThread; ++r) {
      const int p = tid + r * T::kThreads;
      float v = 0.0f;
      if (p < kParams) {
        if (p < kPWs) {
          if (bias != nullptr) {
            const uint16_t h = bias[min(n0 + p, N - 1)];
            v = kF16 ? static_cast<float>(__builtin_bit_cast(_Float16, h)) : __uint_as_float(static_cast<uint32_t>(h) << 16);
          }
        } else if (p < kPAlpha) {
          v = w_scale[min(n0 + (p - kPWs), N - 1)];
        } else {
          v = x_scale[min(m0 + (p - kPAlpha), M - 1)];
          if constexpr (!kRowScale) v = v * *w_scale;
        }
      }
      pv[r] = v;
    }
  };

  // ---- the compute side: current tile (tn, tm), the next (ntn, ntm)
  int tn, tm, ntn = 0, ntm = 0;
  if (!tile_of(0, tn, tm)) return;
  bool more = tile_of(1, ntn, ntm);
  Cursor nxt_ld = more ? cursor_of(ntn, ntm) : cursor_of(tn, tm);
  KFrag f0, f1;
  int g = 0;   // slabs computed so far: the current slab's stage is g & 1

  int ti_par = 0;
  // One slab: all its units, then the slab boundary: wait until the next slab
  // has landed everywhere and everyone is done with this stage, and refill
  // it with the slab after next.  AFTER: a tile's first slab after an
  // epilogue: the wait leaves that epilogue's kStores output stores in flight
  // (they were issued after every load this boundary needs; vector memory
  // counts complete in issue order).  SWITCH (kt = KT - 2): the slab after next is the
  // next tile's first, so the cursor moves to the next tile (after the last
  // tile it stays and re-fetches its own last slab into a stage nobody reads
  // for results).  LAST: the tile's epilogue parameters go to their LDS table
  // before the barrier, and the boundary reads the next tile's first unit.
  auto slab = [&](auto after_c, auto switch_c, auto last_c, auto skip0_c) {
    constexpr bool AFTER = decltype(after_c)::value;
    constexpr bool SWITCH = decltype(switch_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool SKIP0 = decltype(skip0_c)::value;   // unit 0 ran inside the previous epilogue
    const int st = g & 1;
    static_assert(T::kKSteps == 4 || T::kKSteps == 2, "two or four units per slab");
    using L0_ = std::integral_constant<int, 0>;
    read_unit(st, 1, f1);
    if constexpr (!SKIP0) {
      compute_unit(f0);
      order_unit(L0_{});
    }
    if constexpr (T::kKSteps == 4) {
      read_unit(st, 2, f0);
      compute_unit(f1);
      order_unit(L0_{});
      read_unit(st, 3, f1);
      compute_unit(f0);
      order_unit(L0_{});
    }
    if constexpr (LAST && DEQUANT) {
      float* pt = ptab0 + (ti_par & 1) * kParamFloats;
#pragma unroll
      for (int r = 0; r < kParamPerThread; ++r) {
        const int p = tid + r * T::kThreads;
        if (p < kParams) pt[p] = pv[r];
      }
    }
    if constexpr (AFTER) wait_vm_barrier<kStores>();
    else wait_vm_barrier<0>();
    if constexpr (SWITCH) {
      cur_ld = nxt_ld;
      aim(cur_ld);
      ld_kt = more ? 0 : KT - 1;
    }
    issue_loads(st, JA_{}, JE_{});
    ld_kt = min(ld_kt + 1, KT - 1);
    if constexpr (!LAST) read_unit(st ^ 1, 0, f0);
    compute_unit(f1);
    order_boundary(std::integral_constant<bool, !LAST>{});
    ++g;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // ---- prologue: the first tile's first two slabs
  cur_ld = cursor_of(tn, tm);
  aim(cur_ld);
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j) acc[i][j] = acc_t{};
  issue_loads(0, JA_{}, JE_{});
  ld_kt = 1;
  issue_loads(1, JA_{}, JE_{});
  ld_kt = 2;
  if constexpr (DEQUANT) fetch_params(tn * T::BN, tm * T::BM);
  wait_vm_barrier<0>();   // slabs 0 and 1 have landed (the first boundary waits as after an epilogue)
  read_unit(0, 0, f0);
  compute_unit(f0);

  for (int ti = 0;; ++ti) {
    const int n0 = tn * T::BN, m0 = tm * T::BM;
    ti_par = ti;
    // slabs 0 .. KT-1: the first (after an epilogue, or the prologue), plain
    // ones, the cursor's switch at KT - 2, the last
    slab(T_{}, F_{}, F_{}, T_{});
    for (int kt = 1; kt + 2 < KT; ++kt) slab(F_{}, F_{}, F_{}, F_{});
    slab(F_{}, T_{}, F_{}, F_{});
    slab(F_{}, F_{}, T_{}, F_{});
    // ---- epilogue of tile (tn, tm), straight from registers: the last
    // slab's boundary has published this tile's parameter table, and the
    // next tile's first slab has landed in the other stage
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));   // epilogue addressing is not kept live through the loop
    const int lane_e = tid_e & 63;
    const int n_loc = wn * T::kWaveN;
    const bool whole = n0 + T::BN <= N && m0 + T::BM <= M;
    // dequant + bias of four consecutive channels nl.. (tile-relative) of one
    // token, packed in two words
    auto dq4 = [&](const float* pt, float alpha, int nl, const auto& a, int e0, uint32_t (&w)[2]) {
      const float4 b4 = *reinterpret_cast<const float4*>(pt + kPBias + nl);
      const float b[4] = {b4.x, b4.y, b4.z, b4.w};
      float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
      if constexpr (kRowScale) {
        const float4 s4 = *reinterpret_cast<const float4*>(pt + kPWs + nl);
        sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
      }
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (kDefault) v[e] = a[e0 + e] + b[e];
        else if constexpr (kRowScale) v[e] = __builtin_fmaf(static_cast<float>(a[e0 + e]), alpha * sc[e], b[e]);
        else v[e] = __builtin_fmaf(static_cast<float>(a[e0 + e]), alpha, b[e]);
      }
      if constexpr (kF16) {
        // fp16_rne of the fp32 result: no fused fma-and-convert
#pragma unroll
        for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(v[e]));
        w[0] = pack_f16x2(v[0], v[1]);
        w[1] = pack_f16x2(v[2], v[3]);
      } else {
        w[0] = pack_bf16x2(v[0], v[1]);
        w[1] = pack_bf16x2(v[2], v[3]);
      }
    };
    // eight consecutive output channels n.. of token m
    auto put8 = [&](uint16_t* y, int m, int n, const uint4& piece, bool vec) {
      uint16_t* dstp = y + static_cast<int64_t>(m) * N + n;
      if (whole) {
        *reinterpret_cast<uint4*>(dstp) = piece;
      } else if (m < M) {
        if (vec && n + 8 <= N) {
          *reinterpret_cast<uint4*>(dstp) = piece;
        } else {
          const uint32_t w4[4] = {piece.x, piece.y, piece.z, piece.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < N) dstp[e] = static_cast<uint16_t>(w4[e >> 1] >> (16 * (e & 1)));
        }
      }
    };
    // four consecutive int32 results n.. of token m
    auto put4i = [&](int32_t* c, int m, int n, int a0, int a1, int a2, int a3, bool vec) {
      if (m >= M) return;
      int32_t* dstp = c + static_cast<int64_t>(m) * N + n;
      if (vec && n + 3 < N) {
        *reinterpret_cast<int4*>(dstp) = make_int4(a0, a1, a2, a3);
      } else {
        if (n < N) dstp[0] = a0;
        if (n + 1 < N) dstp[1] = a1;
        if (n + 2 < N) dstp[2] = a2;
        if (n + 3 < N) dstp[3] = a3;
      }
    };
    // Result block layout.  32 x 32: lanes 32..63 hold channels 4..7 of each
    // 8.  16 x 16: lane row r (16 lanes) holds channels 4r..4r+3 of token
    // l % 16; v_permlane16_swap of blocks X = (i, j) and Y = (i+1, j) trades
    // rows 1 and 3 of X for rows 0 and 2 of Y, after which lane row r holds
    // channels 8 (r >> 1) + 0..7 of X (r even) or of Y (r odd).
    const int hi = T::MF == 32 ? lane_e >> 5 : lane_e >> 4;
    const int m_loc = wm * T::kWaveM + (lane_e & (T::MF - 1));
    const float* pt = ptab0 + (ti_par & 1) * kParamFloats;
    // dequant epilogue of block (i, j) (32 x 32), or of blocks (i, j) and
    // (i + 1, j) (16 x 16, i even)
    auto epi_block = [&](int i, int j) {
      uint16_t* y = static_cast<uint16_t*>(out);
      const bool vec = (N & 7) == 0;
      const int m = m0 + m_loc + j * T::MF;
      const float alpha = kDefault ? 0.0f : pt[kPAlpha + m_loc + j * T::MF];
      if constexpr (T::MF == 32) {
        uint32_t w[4][2];   // group g: channels 8g + 4*hi + (0..3), packed in pairs
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) dq4(pt, alpha, n_loc + i * 32 + 8 * gg + 4 * hi, acc[i][j], 4 * gg, w[gg]);
        // groups (0,1) and (2,3): lanes l and l+32 trade halves, so lane
        // l < 32 holds channels 16p + 0..7 and lane l + 32 channels 16p + 8..15
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          uint32_t q[4];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const auto r = __builtin_amdgcn_permlane32_swap(w[2 * pp][d], w[2 * pp + 1][d], false, false);
            q[d] = r[0];
            q[2 + d] = r[1];
          }
          put8(y, m, n0 + n_loc + i * 32 + 16 * pp + 8 * hi, make_uint4(q[0], q[1], q[2], q[3]), vec);
        }
      } else {
        uint32_t wx[2], wy[2];
        dq4(pt, alpha, n_loc + i * 16 + 4 * hi, acc[i][j], 0, wx);
        dq4(pt, alpha, n_loc + (i + 1) * 16 + 4 * hi, acc[i + 1][j], 0, wy);
        const auto p0 = __builtin_amdgcn_permlane16_swap(wx[0], wy[0], false, false);
        const auto p1 = __builtin_amdgcn_permlane16_swap(wx[1], wy[1], false, false);
        put8(y, m, n0 + n_loc + 16 * (i + (hi & 1)) + 8 * (hi >> 1), make_uint4(p0[0], p1[0], p0[1], p1[1]), vec);
      }
    };
    constexpr int kIStep = T::MF == 32 ? 1 : 2;
    // A whole tile's dequant epilogue with another tile to follow runs
    // together with that tile's first unit: block by block, the results are
    // converted and stored, and the block's accumulators restart with the
    // next tile's first MFMA (whose fragments are read first: its slab has
    // landed), so the matrix cores work through the epilogue.
    const bool fuse = DEQUANT && whole && more;
    if (fuse) {
      read_unit(g & 1, 0, f0);
#pragma unroll
      for (int j = 0; j < T::TM; ++j)
#pragma unroll
        for (int i = 0; i < T::TN; i += kIStep) {
          epi_block(i, j);
#pragma unroll
          for (int d = 0; d < kIStep; ++d) acc[i + d][j] = mfma<T::MF, OP>(f0.a[i + d], f0.b[j], acc_t{});
          __builtin_amdgcn_sched_barrier(0);
        }
    } else {
      if constexpr (DEQUANT) {
#pragma unroll
        for (int j = 0; j < T::TM; ++j)
#pragma unroll
          for (int i = 0; i < T::TN; i += kIStep) epi_block(i, j);
      } else {
        int32_t* c = static_cast<int32_t*>(out);
        const bool vec = (N & 3) == 0;
        constexpr int kGroups = T::kAccRegs / 4;
#pragma unroll
        for (int i = 0; i < T::TN; ++i)
#pragma unroll
          for (int gg = 0; gg < kGroups; ++gg)
#pragma unroll
            for (int j = 0; j < T::TM; ++j)
              put4i(c, m0 + m_loc + j * T::MF, n0 + n_loc + i * T::MF + 8 * gg + 4 * hi, acc[i][j][4 * gg],
                    acc[i][j][4 * gg + 1], acc[i][j][4 * gg + 2], acc[i][j][4 * gg + 3], vec);
      }
      // the next tile's first boundary leaves kStores stores in flight: that
      // is exact for a whole tile's dequant epilogue; any other epilogue
      // waits for its own stores here
      if (!(DEQUANT && whole)) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (!more) break;
#pragma unroll
      for (int i = 0; i < T::TN; ++i)
#pragma unroll
        for (int j = 0; j < T::TM; ++j) acc[i][j] = acc_t{};
    }
    // ---- on to the next tile (its first slab landed, its second in
    // flight): its parameters, the tile after it for the cursor, and its
    // first unit
    tn = ntn;
    tm = ntm;
    more = tile_of(ti + 2, ntn, ntm);
    nxt_ld = more ? cursor_of(ntn, ntm) : cur_ld;
    if constexpr (DEQUANT) fetch_params(tn * T::BN, tm * T::BM);
    if (!fuse) {
      read_unit(g & 1, 0, f0);
      compute_unit(f0);
    }
  }
}

template <class T, int EPI>
hipError_t launch_tile(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, const uint16_t* bias, void* out, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_n = static_cast<int>((N + T::BN - 1) / T::BN);
  const int tiles_m = static_cast<int>((M + T::BM - 1) / T::BM);
  const int64_t blocks = static_cast<int64_t>(tiles_n) * tiles_m;
  hipLaunchKernelGGL((gemm_i8_kernel<T, EPI>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(T::kThreads), 0, stream, wq, xq, static_cast<int>(M), static_cast<int>(N),
                     static_cast<int>(K), tiles_n, tiles_m, x_scale, w_scale, bias, out);
  return hipGetLastError();
}

// Few-token launch: 16 output channels per workgroup, K split over its four
// waves (M <= 16); the register-streamed kernel where K = 3072 or 4096.
template <int EPI, int S>
hipError_t launch_ksplit(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                         const uint16_t* bias, void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((N + 15) / 16));
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  if (K == 512 * 8)
    hipLaunchKernelGGL((gemm_ksplit_reg_kernel<EPI, 8>), grid, dim3(256), 0, stream, wq, xq, m, n, k, x_scale,
                       w_scale, bias, out);
  else if (K == 512 * 6)
    hipLaunchKernelGGL((gemm_ksplit_reg_kernel<EPI, 6>), grid, dim3(256), 0, stream, wq, xq, m, n, k, x_scale,
                       w_scale, bias, out);
  else
    hipLaunchKernelGGL((gemm_ksplit_kernel<EPI, S>), grid, dim3(256), 0, stream, wq, xq, m, n, k, x_scale, w_scale,
                       bias, out);
  return hipGetLastError();
}

// Persistent launch: one workgroup per CU (at most one per tile).
template <class T, int EPI>
hipError_t launch_persist(const int8_t* xq, const float* x_scale, const int8_t* wq,
                          const float* w_scale, const uint16_t* bias, void* out, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
  const int tiles_n = static_cast<int>((N + T::BN - 1) / T::BN);
  const int tiles_m = static_cast<int>((M + T::BM - 1) / T::BM);
  const int64_t tiles = static_cast<int64_t>(tiles_n) * tiles_m;
  const int64_t grid = tiles < num_cus() ? tiles : num_cus();
  if (K < 3 * T::BK) return launch_tile<T, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  hipLaunchKernelGGL((gemm_persist_kernel<T, EPI>), dim3(static_cast<uint32_t>(grid)), dim3(T::kThreads), 0,
                     stream, wq, xq, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles_n,
                     tiles_m, x_scale, w_scale, bias, out);
  return hipGetLastError();
}

// Tile choice: CONVROT_GEMM_TILE=big|big8|wide|wide128|mid|skinny|skinny16|half|m32|m64|m128|p128|phalf|tall|ptall|ksplit
// forces one (the result does not depend on it; p128, phalf and ptall are the
// persistent 384 x 192, 384 x 96 and 192 x 288 kernels, which take the
// one-tile kernel below three slabs of K; ksplit holds at most 16 tokens).
// Otherwise: M <= 16 streams the weight with the K-split 16 x 16 tile where
// N / 16 is at least twice the CU count, else with the one-wave 16 x 16
// tile, and M <= 256 with the small tile whose
// slowest CU moves the fewest operand bytes; larger layers with fewer
// 384 x 192 tiles than half the CUs use 384 x 96, 128 x 128 or 64 x 128
// tiles.  Else the cost of a large tile is the number of rounds its tiles
// take over the CUs times the work of one tile: 192 x 288 wherever 384 x 192
// would need its half-height tail or costs no less, then the cheaper of
// 384 x 192 and 256 x 256 (the latter only by a clear margin).
int forced_tile() {
  const char* e = getenv("CONVROT_GEMM_TILE");
  if (e == nullptr) return 0;
  if (strcmp(e, "big") == 0) return 1;
  if (strcmp(e, "big8") == 0) return 2;
  if (strcmp(e, "mid") == 0) return 3;
  if (strcmp(e, "wide") == 0) return 4;
  if (strcmp(e, "skinny") == 0) return 5;
  if (strcmp(e, "wide128") == 0) return 6;
  if (strcmp(e, "skinny16") == 0) return 7;
  if (strcmp(e, "half") == 0) return 8;
  if (strcmp(e, "m32") == 0) return 10;
  if (strcmp(e, "m64") == 0) return 11;
  if (strcmp(e, "m128") == 0) return 12;
  if (strcmp(e, "p128") == 0) return 13;
  if (strcmp(e, "phalf") == 0) return 14;
  if (strcmp(e, "tall") == 0) return 15;
  if (strcmp(e, "ptall") == 0) return 16;
  if (strcmp(e, "ksplit") == 0) return 19;
  return 0;
}

int64_t tile_cost(int64_t M, int64_t N, int64_t bn, int64_t bm) {
  const int64_t kCUs = num_cus();
  const int64_t tiles = ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
  return (tiles + kCUs - 1) / kCUs * bn * bm;
}

// Token tiles of 384 x 192 that run in whole rounds.  When their last round
// would be at most half full and the remaining token rows fit one round of
// 384 x 96 tiles, only the whole rounds use 384 x 192 and the rest of M runs
// as half-height tiles; otherwise every token tile is 384 x 192.
int64_t wide_main_m(int64_t M, int64_t N) {
  const int64_t kCUs = num_cus();
  const int64_t tn = (N + 383) / 384, tm = (M + 191) / 192;
  const int64_t tiles = tn * tm, rounds = (tiles + kCUs - 1) / kCUs;
  const int64_t last = tiles - (rounds - 1) * kCUs;
  if (rounds < 2 || 2 * last > kCUs) return tm;
  const int64_t main_m = (rounds - 1) * kCUs / tn;
  const int64_t tail = (M - main_m * 192 + 95) / 96 * tn;
  return main_m > 0 && tail <= kCUs ? main_m : tm;
}

// Cost of 384 x 192 tiles, counting the half-height tail as half a round.
int64_t wide_cost(int64_t M, int64_t N) {
  const int64_t kCUs = num_cus();
  const int64_t tn = (N + 383) / 384, tm = (M + 191) / 192, main_m = wide_main_m(M, N);
  if (main_m == tm) return tile_cost(M, N, 384, 192);
  return ((main_m * tn + kCUs - 1) / kCUs * 2 + 1) * 384 * 96;
}

int pick_tile(int64_t M, int64_t N) {
  const int64_t kCUs = num_cus();
  if (M <= 16) return (N + 15) / 16 >= 2 * kCUs ? 19 : 7;
  if (M <= 256) {
    // Weight-streaming layers.  The slowest CU runs ceil(tiles / CUs) tiles,
    // each moving its BN weight rows and BM token rows per K byte; weight rows
    // count twice (they come from HBM, token rows mostly from L2).  The
    // candidate with the least such traffic wins, ties to the narrower tile.
    // Against the best forced tile on 28 shapes (M = 16..256, N = 3072..12288,
    // K = 3072, weight from HBM): 1.3 % slower on average and 9 % at worst,
    // where a rule by channel count alone was 4 % and 34 %.
    struct Cand { int t, bn, bm; };
    constexpr Cand kCands[] = {{7, 16, 16}, {5, 32, 32}, {10, 64, 32}, {11, 64, 64}, {12, 64, 128}, {3, 128, 128}};
    int best = 7;
    int64_t best_cost = -1;
    for (const Cand& c : kCands) {
      const int64_t tiles = ((N + c.bn - 1) / c.bn) * ((M + c.bm - 1) / c.bm);
      const int64_t cost = (tiles + kCUs - 1) / kCUs * (2 * c.bn + c.bm);
      if (best_cost < 0 || cost < best_cost) best = c.t, best_cost = cost;
    }
    return best;
  }
  // Fewer 384 x 192 tiles than half the CUs: smaller tiles give more
  // workgroups: 384 x 96 when they make one full round (more than 3/8 of the
  // CUs' worth of large tiles: 3072 x 3072 x 3072 in 34.5 us instead of 40.4),
  // else 128 x 128 (two per CU), or 64 x 128 where even those would fill less
  // than half the CUs (weight from HBM: 512 x 12288 x 4096 in 51 us instead of
  // 59, 512 x 3072 x 12288 in 52 instead of 73; from 128 large tiles on,
  // 384 x 192 is faster again: 768 x 12288 x 4096 in 64 us against 76 with
  // 128 x 128)
  const int64_t wide = ((M + 191) / 192) * ((N + 383) / 384);
  if (2 * wide <= kCUs && 8 * wide > 3 * kCUs) return 8;
  if (2 * wide < kCUs)
    return 2 * ((M + 127) / 128) * ((N + 127) / 128) < kCUs ? 12 : 3;
  // 192 x 288 tiles where their rounds cost no more than those of 384 x 192
  // with its tail: with the epilogue run beside the next tile's first MFMAs
  // they are the faster of the two at equal cost (M = 4608, N = 12288,
  // K = 3072: 140.4 us against 145.7; N = 3072 and 9216 take fewer rounds).
  // Where 384 x 192 would need its half-height tail, 192 x 288 tiles are
  // taken at any cost: the tail is a launch of its own whose 384 x 96 tiles
  // run one per workgroup with nothing beside their prologue and epilogue,
  // and it lost on every shape measured (4700 x 12290 x 640: 67 us with
  // 192 x 288 against 80; 16896 x 9216 x 3072: 404 against 427;
  // 19894 x 4096 x 384: 55 against 68).
  if (wide_main_m(M, N) < (M + 191) / 192) return 16;
  if (tile_cost(M, N, 192, 288) <= wide_cost(M, N)) return 16;
  // the 256 x 256 tile (one wave per SIMD) wins only by a clear margin: it
  // was as fast or slower on every shape measured, also where its cost is
  // lower (M = 4608, N = 3072: 184 us for 216 tiles against 180 us for 192 at
  // K = 12288, 57-59 against 52-53 us at K = 3072; 3072 x 9216 x 4096: 142.5
  // against 138.5 us)
  return wide_cost(M, N) * 100 < tile_cost(M, N, 256, 256) * 115 ? 6 : 1;
}

template <int EPI>
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, const uint16_t* bias, void* out, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
  int t = forced_tile();
  const bool automatic = t == 0;
  if (automatic) t = pick_tile(M, N);
  if (t == 1) return launch_tile<TileBig, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 2) return launch_tile<TileBig8, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 4) return launch_tile<TileWide, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 5) return launch_tile<TileSkinny, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (automatic && t == 6) {
    // persistent 384 x 192 tiles where a workgroup gets several (more tiles
    // than CUs) and K has three or more slabs, one-tile workgroups
    // otherwise; both with the half-height tail below
    const int64_t tiles = ((N + 383) / 384) * wide_main_m(M, N);
    if (tiles > num_cus() && K >= 3 * 128) t = 13;
  }
  if (t == 6) {
    // whole rounds of 384 x 192, then (if any) the rest of M as 384 x 96;
    // K counts bytes, and the output rows are 2 (dequant) or 4 (int32) bytes
    const int64_t split = wide_main_m(M, N) * 192;
    if (split >= M) return launch_tile<TileWide128, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
    hipError_t e = launch_tile<TileWide128, EPI>(xq, x_scale, wq, w_scale, bias, out, split, N, K, stream);
    if (e != hipSuccess) return e;
    const int64_t out_elem = EPI == kEpiI32 ? 4 : 2;
    return launch_tile<TileWideHalf, EPI>(xq + split * K, x_scale ? x_scale + split : nullptr, wq, w_scale,
                                          bias, static_cast<char*>(out) + split * N * out_elem, M - split, N,
                                          K, stream);
  }
  if (t == 8) return launch_tile<TileWideHalf, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 13) {
    const int64_t split = wide_main_m(M, N) * 192;
    if (split >= M) return launch_persist<TileWide128, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
    hipError_t e = launch_persist<TileWide128, EPI>(xq, x_scale, wq, w_scale, bias, out, split, N, K, stream);
    if (e != hipSuccess) return e;
    // the tail is at most one round: one tile per workgroup
    const int64_t out_elem = EPI == kEpiI32 ? 4 : 2;
    return launch_tile<TileWideHalf, EPI>(xq + split * K, x_scale ? x_scale + split : nullptr, wq, w_scale, bias,
                                          static_cast<char*>(out) + split * N * out_elem, M - split, N, K, stream);
  }
  if (t == 14) return launch_persist<TileWideHalf, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 15) return launch_tile<TileTall, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 16) return launch_persist<TileTall, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 19 && M > 16) t = 7;   // the K-split tile holds 16 tokens
  if (t == 19) return launch_ksplit<EPI, 2>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 7) return launch_tile<TileSkinny16, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 10) return launch_tile<TileM32, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 11) return launch_tile<TileM64, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  if (t == 12) return launch_tile<TileM128, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
  return launch_tile<TileMid, EPI>(xq, x_scale, wq, w_scale, bias, out, M, N, K, stream);
}

}  // namespace

hipError_t launch_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const uint16_t* bias, uint16_t* y,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_gemm_dequant_ex(xq, x_scale, wq, w_scale, false, bias, y, false, M, N, K, stream);
}

hipError_t launch_gemm_dequant_ex(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, bool row_scale, const uint16_t* bias,
                                  uint16_t* y, bool out_f16, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (out_f16)
    return row_scale ? launch_gemm<kEpiF16Row>(xq, x_scale, wq, w_scale, bias, y, M, N, K, stream)
                     : launch_gemm<kEpiF16>(xq, x_scale, wq, w_scale, bias, y, M, N, K, stream);
  return row_scale ? launch_gemm<kEpiBf16Row>(xq, x_scale, wq, w_scale, bias, y, M, N, K, stream)
                   : launch_gemm<kEpiBf16>(xq, x_scale, wq, w_scale, bias, y, M, N, K, stream);
}

hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M,
                           int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  return launch_gemm<kEpiI32>(xq, nullptr, wq, nullptr, nullptr, acc, M, N, K, stream);
}

hipError_t launch_gemm_default(const uint16_t* x, const uint16_t* wu, const uint16_t* bias, uint16_t* y,
                               bool f16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // operands travel as bytes: a row of K 16-bit values is 2K bytes
  const auto* a = reinterpret_cast<const int8_t*>(x);
  const auto* b = reinterpret_cast<const int8_t*>(wu);
  return f16 ? launch_gemm<kEpiDefF16>(a, nullptr, b, nullptr, bias, y, M, N, 2 * K, stream)
             : launch_gemm<kEpiDefBf16>(a, nullptr, b, nullptr, bias, y, M, N, 2 * K, stream);
}

}  // namespace convrot
