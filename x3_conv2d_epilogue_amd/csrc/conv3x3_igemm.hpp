// conv3x3_igemm.hpp -- fused valid 3x3 convolution (stride 1, bias) as an
// im2col-free implicit GEMM on the gfx950 fp32 matrix cores, with the
// epilogue applied in registers.
//
// GEMM view (per sample n):
//   C[co][p] = b[co] + sum_k A[co][k] * B[k][p]
//   A[co][k] = w[co][ci][kh][kw],  B[k][p] = x[n][ci][r+kh][c+kw],
//   p = (r, c) an output pixel, k = (ci, kh, kw).
// B is never materialised: it is read out of an LDS copy of the input tile
// plus its 2-row/2-column halo (the staging idea discussed in the
// POPCORNBENCH l2_p54 transcript, where an input tile and a weight tile are
// kept in shared memory).
//
// Work decomposition
//   * A workgroup tile is TH output rows x TWC = 32*NCT output columns of one
//     sample, and ALL output channels, so channel reductions (the min
//     epilogues) never leave the workgroup -- they never leave the
//     wavefront, in fact.  The channels are covered by ncb passes over
//     channel blocks of COUT = 32*MT; the last block is padded with zero
//     weight rows (and, for the channel-min epilogues, with a bias of
//     +-infinity, so a padded channel never wins).  The min epilogues carry
//     a running per-pixel extremum in registers from pass to pass.
//   * The tile is split into 32x32 MFMA blocks: M = 32 channels, N = 32
//     consecutive pixels of one output row.  Each of the NWAVE wavefronts
//     owns all MT channel blocks for NW pixel blocks ("N-tiles") that sit in
//     one 32-column strip, NW consecutive rows.
//   * K is walked in chunks of CC input channels (K-chunk = 9*CC).  A chunk's
//     input tile and weight tile are copied HBM/L2 -> LDS by direct-to-LDS
//     buffer loads (no VGPR staging) into one of two LDS stages while the
//     matrix cores work on the other stage.
//   * The kernel is persistent: a grid of about one workgroup per CU walks a
//     flat stream of (tile, chunk) items, so the first chunk of the next tile
//     is already in flight while the current tile finishes and runs its
//     epilogue.
//
// MFMA v_mfma_f32_32x32x2_f32 operand layout (wave64):
//   A (32x2): lane l supplies A[m = l%32][k = l/32]
//   B (2x32): lane l supplies B[k = l/32][n = l%32]
//   C (32x32): lane l, accumulator element i holds
//              C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32]
// K order inside a chunk: k-step s (two k values per MFMA) is
//   s = tap*(CC/2) + cp, tap = kh*3+kw; lane half h = l/32 takes input
//   channel ci = 2*cp + h.  With this order every LDS address is a per-lane
//   base plus a compile-time immediate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "epi_math.hpp"

namespace x3 {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define X3_LDS __attribute__((address_space(3)))
// Every helper lambda of the kernel must inline: they capture the
// accumulator array by reference, and an out-of-line call would force it
// into scratch memory.
#define X3_INLINE __attribute__((always_inline))

enum Epilogue : int {
  EPI_MIN_TANH2 = 0,       // tanh(tanh(min_co y))
  EPI_MUL_LRELU_GELU = 1,  // exact GELU(LeakyReLU(y * mult[co]))
  EPI_SCALE_MIN = 2,       // min_co(scale * y)
  EPI_GN_POOL = 3,         // GroupNorm partials per group of 4 channels
                           // + pooling-window extrema
  EPI_GN_POOL_CH = 4,      // GroupNorm partials per channel (any group
                           // size) + pooling-window extrema
  EPI_STORE = 5,           // the conv output itself (split path)
  EPI_MUL_LRELU_GELU_TANH = 6,  // tanh-form GELU(LeakyReLU(y * mult[co]))
  EPI_GN_POOLK = 7,        // GroupNorm partials per group of 4 channels +
                           // extrema of pooling windows of size 1 or 2
  EPI_GN_POOLK_CH = 8,     // per-channel partials + windows of size 1 or 2
  EPI_GN_POOLKL = 9        // per-channel partials + windows of size 3..16,
                           // combined across wavefronts in LDS
};

// Kernel arguments (plain values, passed by value).
struct ConvArgs {
  const float* x;
  const float* w;
  const float* b;
  float* out;
  const float* v0;  // mult (EPI_MUL_LRELU_GELU*) | gamma (EPI_GN_POOL*)
  const float* v1;  // beta  (EPI_GN_POOL*)
  const float* v2;  // scale (EPI_GN_POOL*)
  float s0;         // neg_slope (EPI_MUL_LRELU_GELU*) | scale (EPI_SCALE_MIN)
  float4* part;     // GroupNorm partials (EPI_GN_POOL*)
  int B, Cin, H, W, Cout;
  int Ho, Wo;
  int n_rt, n_ct;   // row tiles, column tiles per sample
  int ntiles;       // B * n_rt * n_ct
  int nchunk;       // ceil(Cin / CC)
  int ncb;          // channel-block passes per tile: ceil(Cout / COUT)
  int Ph, Pw;       // pooled output size (EPI_GN_POOL*)
  int groups;       // GroupNorm groups (EPI_GN_POOL*)
  int flags;        // kOutVec4: NHWC out takes 16-byte stores (Cout % 4
                    // == 0 and out 16-byte aligned)
  int pk;           // pooling window (EPI_GN_POOLK*)
  int thk, twk;     // output rows / columns a tile covers (set by the
                    // launcher: TH x TWC, or for EPI_GN_POOLK* the largest
                    // multiples of the window that fit, so that no window
                    // crosses a tile)
};

constexpr int kOutVec4 = 1;

// Largest Cout: per-channel constants of all channel blocks live in LDS.
constexpr int kMaxCout = 1024;

// Pooling windows other than 4x4 (EPI_GN_POOLK*): sizes 1 and 2 fold
// inside a wavefront; sizes 3..16 are combined across the wavefronts of a
// tile in LDS, where a tile of TH x TWC outputs holds at most (TH/3) x
// (TWC/3) windows.  (Separate kernels: with all three forms, or with
// group-of-4 partials next to the LDS window buffer, the kernel needs more
// than the 256 registers of two waves per SIMD.)
template <int EPI>
constexpr bool gn_generic_k() {
  return EPI == EPI_GN_POOLK || EPI == EPI_GN_POOLK_CH || EPI == EPI_GN_POOLKL;
}
template <int EPI>
constexpr bool gn_epilogue() {
  return EPI == EPI_GN_POOL || EPI == EPI_GN_POOL_CH || gn_generic_k<EPI>();
}

// Compile-time geometry of one kernel configuration.
template <int MT_, int CC_, int TH_, int NCT_, int NWAVE_, bool X4_,
          int RC_ = 0, bool NHWC_ = false>
struct Geo {
  static constexpr int MT = MT_;          // 32-channel MFMA blocks per pass
  static constexpr int CC = CC_;          // input channels per K chunk
  static constexpr int TH = TH_;          // output rows per tile
  static constexpr int NCT = NCT_;        // 32-column strips per tile
  static constexpr int NWAVE = NWAVE_;
  // Input rows are 16-byte aligned in memory (W % 4 == 0): stage the input
  // with 16-byte-per-lane loads (4x fewer load instructions).
  static constexpr bool X4 = X4_;
  // RC > 0: the weight tiles of all K chunks (at most RC of them, one
  // channel block) stay resident in LDS for the whole kernel; items then
  // stage the input only.
  static constexpr int RC = RC_;
  static constexpr bool RESW = RC > 0;
  // x (and the per-channel outputs) in NHWC order.
  //  * 4-byte staging: the input tile is staged pixel-major,
  //    [XROWS][XCOLS][CCP], CCP = CC + 2.  With a pitch of 2 mod 4 dwords
  //    per pixel, the 32 pixels x 2 adjacent channels of a B-fragment read
  //    (lane half h reads channel 2cp + h) fall in 64 distinct banks.
  //  * NH4, 16-byte staging (Cin % 4 == 0): pixel-major, [XROWS][XCOLS][2]
  //    slots of 4 channels; slot s of the pixel in column col holds channels
  //    4(s ^ b3) .. 4(s ^ b3) + 3 of the chunk, b3 = bit 3 of col.  Two
  //    adjacent lanes stage one pixel's 32 contiguous bytes, so a load
  //    instruction touches 32 lines of x where separate channel-half
  //    regions touched 64.  K order: k-step s takes tap s/4, and lane half
  //    h channel 4h + s%4, so a lane's B values of the 4 k-steps of a tap
  //    are one ds_read_b128 (slot h ^ b3); 16 consecutive columns at an
  //    8-dword pitch cover all 64 banks, as columns 8 apart use opposite
  //    slots.
  static constexpr bool NHWC = NHWC_;
  static constexpr bool NH4 = NHWC_ && X4_;
  static constexpr int CCP = CC + 2;
  static constexpr int NTHR = NWAVE * 64;
  static constexpr int COUT = 32 * MT;    // channels per pass
  static constexpr int TWC = 32 * NCT;    // output columns per tile
  static constexpr int XROWS = TH + 2;    // input rows per tile (halo)
  static constexpr int XCOLS = TWC + 2;   // input columns per tile (halo)
  static constexpr int XP = (XCOLS + 3) / 4 * 4;  // LDS row pitch (dwords)
  // K order inside a chunk.
  //  * KO (the 16-byte configurations, NCHW): k-step s = 0..KS-1 and lane
  //    half h take K index s + KS*h, i.e. channel s/9 + CC/2*h at tap s%9.
  //    A lane's weights for 4 consecutive k-steps are then 4 consecutive
  //    floats of its weight row (one ds_read_b128), and weight rows are
  //    staged with 16-byte loads (pitch WP = 76: 16-byte aligned rows, and
  //    76 = 12 mod 64 puts 16 consecutive rows in 16 disjoint 4-bank
  //    groups).  The input channel stride CS = 8 mod 16 makes the two
  //    halves' channels (CC/2 = 4 apart) fall in opposite bank halves.
  //  * otherwise: k-step s = tap*(CC/2) + cp, lane half h takes channel
  //    2*cp + h; channel stride CS = 32 mod 64 (opposite bank halves for
  //    adjacent channels), odd weight pitch WP = KC + 1 (conflict-free
  //    4-byte reads).
  static constexpr bool KO = X4 && !NHWC;
  static constexpr int PXS = XROWS * XCOLS * 8;  // NH4: dwords of the pixel slots
  static constexpr int CS0 = XROWS * XP;
  static constexpr int CS =
      KO ? CS0 + ((8 - (CS0 % 16)) + 16) % 16
         : CS0 + ((32 - (CS0 % 64)) + 64) % 64;
  static constexpr int KC = 9 * CC;       // K per chunk
  static constexpr int XBLK = X4 ? 256 : 64;
  static constexpr int XBUF =             // input dwords per stage
      NH4    ? (PXS + 255) / 256 * 256
      : NHWC ? (XROWS * XCOLS * CCP + 63) / 64 * 64
             : (CC * CS + XBLK - 1) / XBLK * XBLK;
  // weight-row pitch: 16-byte staged rows (KO and NH4) as described for KO
  static constexpr int WP = X4 ? KC + 4 : KC + 1;
  static constexpr int WBUF = COUT * WP;  // weight dwords per stage
  // Staging blocks: the input region is filled in blocks of 256 dwords
  // (16 bytes per lane, X4) or 64 dwords (4 bytes per lane), the weight
  // region likewise (256 with KO).  Every wavefront issues the same number
  // of blocks, NBI + NBW per item; a wavefront whose turn runs past the
  // last block reloads the last block (same data to the same place).
  static constexpr int WBLK = X4 ? 256 : 64;
  static constexpr int NBX = XBUF / XBLK;                 // input blocks
  static constexpr int NBWT = WBUF / WBLK;                // weight blocks
  static constexpr int NBI = (NBX + NWAVE - 1) / NWAVE;   // per wave
  static constexpr int NBW = (NBWT + NWAVE - 1) / NWAVE;  // per wave
  static constexpr int STAGE = XBUF + (RESW ? 0 : WBUF);
  static constexpr int LDS_DWORDS = 2 * STAGE + RC * WBUF;
  static constexpr int KS = KC / 2;       // MFMA k-steps per chunk
  static constexpr int NTILE_N = TH * NCT;  // N-tiles per workgroup tile
  static constexpr int NW = NTILE_N / NWAVE;  // N-tiles per wave

  static_assert(CC % 2 == 0, "CC must be even");
  static_assert(!NHWC || CC % 4 == 0, "NHWC: CC % 4 == 0 (pitch 2 mod 4)");
  static_assert(!NH4 || (CC == 8 && KS % 4 == 0), "NH4: 8-channel chunks");
  static_assert(XBUF % XBLK == 0 && WBUF % WBLK == 0, "whole staging blocks");
  static_assert(!KO || (CC == 8 && KS % 4 == 0 && (CC / 2 * CS) % 64 == 32),
                "KO: 8-channel chunks, halves in opposite bank halves");
  static_assert(NTILE_N % NWAVE == 0, "N-tiles must split evenly over waves");
  static_assert(TH % NW == 0, "a wave's N-tiles must lie in one strip");
  static_assert(LDS_DWORDS * 4 + 2 * kMaxCout * 4 <= 160 * 1024,
                "LDS budget exceeded");
  static_assert(XBUF * 4 < 65536 && WBUF * 4 < 65536,
                "ds_read immediates are 16-bit");
};

// ---------------------------------------------------------------------------
// small device helpers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  // Raw (un-strided) buffer: offsets >= `bytes` read as zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)bytes, 0x00020000);
}

// 16-byte-per-lane direct-to-LDS load.  The size-16 form exists only on
// gfx950, so only the device compilation pass may see the builtin (the host
// pass would otherwise drop the kernels that use it).
__device__ __forceinline__ void lds_load_x4(__amdgpu_buffer_rsrc_t r,
                                            X3_LDS void* dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
#endif
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// DPP lane permutations (within rows of 16 lanes), applied to a float.
enum : int {
  DPP_QUAD_XOR1 = 0xB1,  // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,  // quad_perm [2,3,0,1]
  DPP_ROW_MIRROR = 0x140,       // lane i of a row of 16 <- lane 15 - i
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i of a half-row of 8 <- lane 7 - i
  DPP_ROW_ROR4 = 0x124,  // rotate a row of 16 by 4
  DPP_ROW_ROR8 = 0x128   // rotate a row of 16 by 8
};
// (All of them stay inside a row, so no lane reads a disabled source; the
// bound-control form needs no register for the unused `old` operand.)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, true));
}
// NaN-propagating maximum / minimum (v_maximum3_f32 / v_minimum3_f32 on
// gfx950: two inputs per instruction in a chain, and no quieting of the
// inputs, which fmaxf / fminf need in IEEE mode for values the compiler
// cannot prove quiet, such as matrix-core results and lane permutations).
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float vmin(float a, float b) {
  return __builtin_elementwise_minimum(a, b);
}
// Lane l <-> l ^ 16 inside each half-wave (ds_swizzle bit mode:
// and_mask 0x1F, xor_mask 0x10).
__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
// The value lane 0 holds (for lanes 0..31) or lane 32 holds (lanes 32..63):
// a bit-mode swizzle with all masks zero reads lane 0 of each 32-lane half
// (one LDS-pipe instruction instead of two readlanes and a select).  Every
// lane must be active, as everywhere in the epilogues.
__device__ __forceinline__ float half_lane0(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x0000));
}
// Sum over the 32 lanes of a half-wave, returned to every lane of it.
__device__ __forceinline__ float sum32(float v) {
  v += dpp<DPP_QUAD_XOR1>(v);
  v += dpp<DPP_QUAD_XOR2>(v);
  v += dpp<DPP_ROW_ROR4>(v);
  v += dpp<DPP_ROW_ROR8>(v);
  return v + swz_xor16(v);
}

// Row r of the output tile stored by the wave's N-tile j, etc.
template <class G>
struct WaveMap {
  int strip;    // 32-column strip index inside the tile
  int row0;     // first row (inside the tile) of the wave's N-tiles
  __device__ __forceinline__ explicit WaveMap(int wave) {
    const int first = wave * G::NW;  // N-tile index, strip-major
    strip = first / G::TH;
    row0 = first % G::TH;
  }
};

// ---------------------------------------------------------------------------
// The kernel.

template <class G, int EPI>
__global__ void __launch_bounds__(G::NTHR)
    __attribute__((amdgpu_waves_per_eu(2, 2)))
    conv3x3_igemm_kernel(const ConvArgs a) {
  // Two LDS stages as two separate arrays: the direct-to-LDS loads that
  // fill one stage are then visibly disjoint from the fragment reads of the
  // other, so no wait is needed between them inside the MFMA loop.
  // (16-byte aligned: direct-to-LDS 16-byte staging, ds_read_b128)
  __shared__ __attribute__((aligned(16))) float lds0[G::STAGE];
  __shared__ __attribute__((aligned(16))) float lds1[G::STAGE];
  __shared__ __attribute__((aligned(16)))
  float ldsw[G::RESW ? G::RC * G::WBUF : 1];  // resident weights
  // Per-channel constants of all ncb*COUT (padded) channels, loaded once:
  // bias, and the epilogue's channel parameter (multiplier, or for the
  // pooling path the direction +1 = keep the window maximum, -1 = keep the
  // minimum).  Reading them from LDS keeps global loads out of the main
  // loop, whose vmcnt waits would otherwise also wait for the next stage's
  // prefetch.
  __shared__ float s_bias[kMaxCout];
  __shared__ __attribute__((aligned(16))) float s_par[kMaxCout];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;     // lane half
  const int l32 = lane & 31;   // column inside an N-tile

  // Persistent schedule, XCD aware: consecutive workgroup ids are spread
  // round-robin over the 8 XCDs, so renumber them so that the workgroups
  // resident on one XCD work on neighbouring tiles (shared halo rows and
  // the same weights stay in that XCD's L2).
  const int G_ = gridDim.x;
  int vb = blockIdx.x;
  if ((G_ & 7) == 0) vb = (blockIdx.x & 7) * (G_ >> 3) + (blockIdx.x >> 3);
  const int my_tiles = (a.ntiles > vb) ? (a.ntiles - vb + G_ - 1) / G_ : 0;
  const int nitems = my_tiles * a.ncb * a.nchunk;

  const uint32_t x_sample = (uint32_t)a.Cin * a.H * a.W;  // floats
  constexpr bool PRE = G::X4;  // precomputed staging offsets (see below)
  const uint32_t w_total = (uint32_t)a.Cout * a.Cin * 9u;  // floats

  // ---- staging of one (tile, chunk) item ------------------------------------
  // The stage is filled in blocks, one direct-to-LDS load per block and
  // wave (lane l writes piece l of the block).  Wave w owns input blocks
  // w + NWAVE*i (i < NBI) and weight blocks w + NWAVE*i (i < NBW).
  // PRE (the 16-byte configurations, NCHW and NHWC): a wave stages the same
  // blocks of every item's tile, so the per-lane part of each block's
  // source offset is computed once (xoff, woff); the item's position goes
  // into the buffer resources, which are scalars, so the staging costs
  // almost no vector instructions per item.  Rows past H and columns past W
  // are not masked: they read the data that follows in the sample (values
  // that reach only conv outputs outside the image, which are neither
  // stored nor counted) or lie past its end and read as 0.  Input channels
  // past Cin read as 0 too: in NCHW they start past the end of the sample;
  // in NHWC (Cin % 8 == 4: the upper half of a last chunk) their pieces
  // take offsets with the drop bit (xoffh).  Weight columns past the chunk's
  // K are masked.  The other configurations (4 times as many blocks, too
  // many registers to keep) compute masked offsets per item: rows past H,
  // input channels past Cin and weight columns past the chunk's K read as
  // 0.  Either way the weight rows of padded output channels lie past the
  // end of the weight tensor by construction and read as 0.
  //
  // Items run tile by tile; inside a tile, channel block by channel block;
  // inside a block, K chunk by K chunk.  A position in that walk is
  // advanced incrementally (no integer division per item).
  struct Pos {
    int tl, cb, chunk;  // local tile index, channel block, K chunk
  };
  auto advance = [&](const Pos& p) X3_INLINE {
    const bool end_k = p.chunk + 1 == a.nchunk;
    const bool end_c = end_k && (p.cb + 1 == a.ncb);
    Pos q;
    q.chunk = end_k ? 0 : p.chunk + 1;
    q.cb = end_c ? 0 : (end_k ? p.cb + 1 : p.cb);
    q.tl = end_c ? p.tl + 1 : p.tl;
    return q;
  };
  struct Item {
    int n, r0, c0, ci0, co0;
  };
  auto item_of = [&](const Pos& p) X3_INLINE {
    const int t = vb + p.tl * G_;
    const int chunk = p.chunk, cb = p.cb;
    const int ct = t % a.n_ct;
    const int rt = (t / a.n_ct) % a.n_rt;
    Item it;
    it.n = t / (a.n_ct * a.n_rt);
    it.r0 = rt * a.thk;
    it.c0 = ct * a.twk;
    it.ci0 = chunk * G::CC;
    it.co0 = cb * G::COUT;
    return it;
  };
  // Uniform per-item limits, computed once per item.
  struct Lim {
    __amdgpu_buffer_rsrc_t xr;  // PRE: based at the item's first element
    __amdgpu_buffer_rsrc_t wr;  // PRE: based at the item's first weight
    int base;      // element offset of (ci0, r0, c0) in the sample
    int ci_lim;    // masked staging (not PRE): local channels < ci_lim
    int row_lim;   //   (NHWC: and < CC), rows < row_lim and columns <
    int col_lim;   //   col_lim are real
    int kk_lim;    // weight columns < kk_lim are real
    int wbase;     // element offset of (co0, ci0) in the weight tensor
    int wslot;     // resident weights: the chunk's slot in ldsw
  };
  const int HW = a.H * a.W, CinK = a.Cin * 9;
  auto lim_of = [&](const Item& it) X3_INLINE {
    Lim l;
    if constexpr (G::NH4) {
      l.base = (it.r0 * a.W + it.c0) * a.Cin + it.ci0;
      l.xr = make_rsrc(a.x + (size_t)it.n * x_sample + l.base,
                       (x_sample - (uint32_t)l.base) * 4u);
      l.ci_lim = a.Cin - it.ci0;
    } else if constexpr (G::NHWC) {
      l.xr = make_rsrc(a.x + (size_t)it.n * x_sample, x_sample * 4u);
      l.base = (it.r0 * a.W + it.c0) * a.Cin + it.ci0;
      const int cl = a.Cin - it.ci0;
      l.ci_lim = cl < G::CC ? cl : G::CC;
    } else if constexpr (PRE) {
      l.base = (it.ci0 * a.H + it.r0) * a.W + it.c0;
      l.xr = make_rsrc(a.x + (size_t)it.n * x_sample + l.base,
                       (x_sample - (uint32_t)l.base) * 4u);
    } else {
      l.xr = make_rsrc(a.x + (size_t)it.n * x_sample, x_sample * 4u);
      l.base = (it.ci0 * a.H + it.r0) * a.W + it.c0;
      l.ci_lim = a.Cin - it.ci0;
    }
    const int rl = a.H - it.r0;
    l.row_lim = rl < G::XROWS ? rl : G::XROWS;
    const int cl = a.W - it.c0;
    l.col_lim = cl < G::XCOLS ? cl : G::XCOLS;
    const int kl = 9 * (a.Cin - it.ci0);
    l.kk_lim = kl < G::KC ? kl : G::KC;
    l.wbase = it.co0 * CinK + it.ci0 * 9;
    l.wr = PRE ? make_rsrc(a.w + l.wbase, (w_total - (uint32_t)l.wbase) * 4u)
               : make_rsrc(a.w, w_total * 4u);
    l.wslot = 0;
    return l;
  };
  // Per-lane staging offsets (bytes) of the wave's input and weight
  // blocks; bit 31 set = never loaded (stage padding past CC channels,
  // weight-row padding past K).
  uint32_t xoff[PRE ? G::NBI : 1];
  // NH4 weight rows in the order the K walk reads them (PW): a weight row
  // holds K index (4h + e)*9 + tap at dword 36h + 4*tap + e, so a lane's
  // weights for the 4 k-steps of a tap are 4 consecutive dwords (one
  // conflict-free ds_read_b128, as in KO).  The permutation moves single
  // floats, so those rows are staged with 4-byte loads, NBWP blocks of 64
  // dwords per wave, each with its per-lane source offset kept in a
  // register while the weights are staged per item.  Taken with resident
  // weights (staged once) and with 64-channel blocks; 128-channel blocks
  // staged per item read the unpermuted rows with 4-byte fragment reads
  // (their 19 four-byte weight loads per wave and item cost more than the
  // bank conflicts they remove), and so do the pooling-window epilogues
  // with staged weights (no registers left for the offsets).
  constexpr bool PW =
      G::NH4 && (G::RESW || (G::MT == 2 && !gn_generic_k<EPI>()));
  constexpr int NBWTP = G::WBUF / 64;                     // 4-byte weight blocks
  constexpr int NBWP = (NBWTP + G::NWAVE - 1) / G::NWAVE;  // per wave
  constexpr int NBWK = PW ? NBWP : G::NBW;  // weight blocks per wave
  uint32_t woff[PRE ? NBWK : 1], wkk[PRE && !PW ? G::NBW : 1];
  // NH4: the same offsets with the pieces of the upper channel half
  // dropped, for a last chunk of 4 channels (Cin % 8 == 4)
  uint32_t xoffh[G::NH4 ? G::NBI : 1];
  if constexpr (G::NH4) {
#pragma unroll
    for (int i = 0; i < G::NBI; ++i) {
      int blk = wave + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      // lane l moves slot sl of pixel pc: channels 4*hc .. 4*hc + 3, hc =
      // sl ^ (bit 3 of the pixel's column); pieces past the tile's pixels
      // (stage padding) are not loaded
      const uint32_t P = (uint32_t)(blk * 64 + lane);
      const uint32_t pc = P >> 1;
      const uint32_t row = pc / G::XCOLS;
      const uint32_t col = pc - row * G::XCOLS;
      const uint32_t hc = (P & 1u) ^ ((col >> 3) & 1u);
      xoff[i] = (((row * (uint32_t)a.W + col) * (uint32_t)a.Cin + 4u * hc) << 2) |
                ((uint32_t)(pc >= (uint32_t)(G::XROWS * G::XCOLS)) << 31);
      xoffh[i] = xoff[i] | (hc << 31);
    }
  } else if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < G::NBI; ++i) {
      int blk = wave + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      // first dword of this lane's piece; with X4 the lane moves 4
      // consecutive dwords of one row (XP and CS are multiples of 4, so a
      // piece never crosses a row)
      const uint32_t p = (uint32_t)(blk * G::XBLK + lane * (G::XBLK / 64));
      const uint32_t cil = p / G::CS;
      const uint32_t rem = p - cil * G::CS;
      const uint32_t row = rem / G::XP;
      const uint32_t col = rem - row * G::XP;
      xoff[i] = ((cil * (uint32_t)HW + row * (uint32_t)a.W + col) << 2) |
                ((uint32_t)(cil >= (uint32_t)G::CC) << 31);
    }
  }
  if constexpr (PW) {
#pragma unroll
    for (int i = 0; i < NBWP; ++i) {
      int blk = wave + i * G::NWAVE;
      blk = blk < NBWTP - 1 ? blk : NBWTP - 1;
      // LDS dword j of row co <- K index (4h + e)*9 + tap; dwords past the
      // 72 of a row are padding (read as zero); bit 30 marks the upper
      // channel half, which a last chunk of 4 channels masks
      const uint32_t q = (uint32_t)(blk * 64 + lane);
      const uint32_t co = q / G::WP;
      const uint32_t j = q - co * G::WP;
      const uint32_t hh = j >= (uint32_t)G::KS;
      const uint32_t r = j - hh * (uint32_t)G::KS;
      const uint32_t kk = (4u * hh + (r & 3u)) * 9u + (r >> 2);
      woff[i] = ((co * (uint32_t)CinK + kk) << 2) | (hh << 30) |
                ((uint32_t)(j >= (uint32_t)G::KC) << 31);
    }
  } else if constexpr (PRE) {
#pragma unroll
    for (int i = 0; i < G::NBW; ++i) {
      int blk = wave + i * G::NWAVE;
      blk = blk < G::NBWT - 1 ? blk : G::NBWT - 1;
      // lane l moves 4 consecutive floats of one weight row (the pitch
      // and the row's K columns are multiples of 4; the dispatch keeps
      // Cin % 4 == 0 so the global rows are 16-byte aligned too)
      const uint32_t q = (uint32_t)(blk * G::WBLK + lane * (G::WBLK / 64));
      const uint32_t co = q / G::WP;
      const uint32_t kk = q - co * G::WP;
      wkk[i] = kk;
      woff[i] = ((co * (uint32_t)CinK + kk) << 2) |
                ((uint32_t)(kk >= (uint32_t)G::KC) << 31);
    }
  }
  // Wave-local block i (compile-time) of the stage at `sbase`.  An element
  // that must read as zero gets bit 31 set in its offset: every buffer here
  // is smaller than 2 GiB, so such an offset is past num_records and the
  // load returns 0.  (An OR rather than a select keeps the compiler from
  // turning this into an exec-masked region.)  Without PRE the offsets are
  // computed per item, masked; `zz` is an opaque per-item zero that keeps
  // that lane-dependent arithmetic from being hoisted out of the item loop
  // (which would pin one register per block for the whole kernel).
  auto issue = [&](const Lim& l, X3_LDS float* sbase, int i, int zz)
                   X3_INLINE {
    if (i < G::NBI && G::NH4) {
      int blk = wave + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      // (uniform) a last chunk with 4 channels: its upper half reads 0
      lds_load_x4(l.xr, (X3_LDS void*)(sbase + blk * 256),
                  l.ci_lim <= 4 ? xoffh[i] : xoff[i]);
    } else if (i < G::NBI && G::NHWC) {
      int blk = wave + zz + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      // LDS dword p of the tile is (pixel p / CCP, channel slot p % CCP);
      // slots >= CC are padding, read as zero.  Consecutive lanes walk the
      // channels of one pixel, then the next pixel of the row.
      const uint32_t p = (uint32_t)(blk * 64 + lane);
      const uint32_t pix = p / G::CCP;
      const uint32_t slot = p - pix * G::CCP;
      const uint32_t row = pix / G::XCOLS;
      const uint32_t col = pix - row * G::XCOLS;
      const bool ok = (slot < (uint32_t)l.ci_lim) &
                      (row < (uint32_t)l.row_lim) &
                      (col < (uint32_t)l.col_lim);
      const uint32_t off =
          (((row * (uint32_t)a.W + col) * (uint32_t)a.Cin + slot +
            (uint32_t)l.base) << 2) | ((uint32_t)!ok << 31);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          l.xr, (X3_LDS void*)(sbase + blk * 64), 4, off, 0, 0, 0);
    } else if (i < G::NBI && PRE) {
      int blk = wave + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      lds_load_x4(l.xr, (X3_LDS void*)(sbase + blk * G::XBLK), xoff[i]);
    } else if (i < G::NBI) {
      int blk = wave + zz + i * G::NWAVE;
      blk = blk < G::NBX - 1 ? blk : G::NBX - 1;
      const uint32_t p = (uint32_t)(blk * G::XBLK + lane * (G::XBLK / 64));
      const uint32_t cil = p / G::CS;
      const uint32_t rem = p - cil * G::CS;
      const uint32_t row = rem / G::XP;
      const uint32_t col = rem - row * G::XP;
      const bool ok = (cil < (uint32_t)l.ci_lim) &
                      (row < (uint32_t)l.row_lim) &
                      (col < (uint32_t)l.col_lim);
      const uint32_t off =
          ((cil * (uint32_t)HW + row * (uint32_t)a.W + col +
            (uint32_t)l.base) << 2) | ((uint32_t)!ok << 31);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          l.xr, (X3_LDS void*)(sbase + blk * G::XBLK), 4, off, 0, 0, 0);
    } else if constexpr (PW) {
      const int iw = i - G::NBI;
      int blk = wave + iw * G::NWAVE;
      blk = blk < NBWTP - 1 ? blk : NBWTP - 1;
      X3_LDS float* wdst =
          G::RESW ? (X3_LDS float*)ldsw + l.wslot * G::WBUF : sbase + G::XBUF;
      // (Cin % 4 == 0: a short last chunk has 4 channels, K = 36)
      const uint32_t hi = (woff[iw] >> 30) & 1u;
      const uint32_t off = (woff[iw] & ~(1u << 30)) |
                           ((hi & (uint32_t)(l.kk_lim <= G::KS)) << 31);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          l.wr, (X3_LDS void*)(wdst + blk * 64), 4, off, 0, 0, 0);
    } else {
      const int iw = i - G::NBI;
      int blk = wave + (PRE ? 0 : zz) + iw * G::NWAVE;
      blk = blk < G::NBWT - 1 ? blk : G::NBWT - 1;
      X3_LDS float* wdst =
          G::RESW ? (X3_LDS float*)ldsw + l.wslot * G::WBUF : sbase + G::XBUF;
      X3_LDS void* dst = (X3_LDS void*)(wdst + blk * G::WBLK);
      if constexpr (PRE) {
        // columns past the chunk's K (a last chunk of fewer than CC
        // channels) read as zero
        const uint32_t off =
            woff[iw] | ((uint32_t)(wkk[iw] >= (uint32_t)l.kk_lim) << 31);
        lds_load_x4(l.wr, dst, off);
      } else {
        const uint32_t q = (uint32_t)(blk * G::WBLK + lane);
        const uint32_t co = q / G::WP;
        const uint32_t kk = q - co * G::WP;
        const bool ok = kk < (uint32_t)l.kk_lim;
        const uint32_t off =
            ((co * (uint32_t)CinK + (uint32_t)l.wbase + kk) << 2) |
            ((uint32_t)!ok << 31);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(l.wr, dst, 4, off, 0, 0, 0);
      }
    }
  };

  // blocks per wave per item, BPS per k-step over the first half of the
  // k-steps, so that they have the second half to land
  constexpr int NB_W = G::NBI + (G::RESW ? 0 : NBWK);
  constexpr int KS_ISSUE = G::KS / 2 > 0 ? G::KS / 2 : 1;
  constexpr int BPS = (NB_W + KS_ISSUE - 1) / KS_ISSUE;

  const WaveMap<G> wm(wave);

  // Padded channels (co >= Cout) get the bias that loses every channel
  // comparison: +inf for a minimum, -inf for a maximum (scale_min with a
  // negative scale takes the maximum before scaling); their weight rows are
  // zero, so the accumulator stays at that bias.  Other epilogues never
  // store padded channels.
  float pad = 0.0f;
  if constexpr (EPI == EPI_MIN_TANH2) pad = __builtin_inff();
  if constexpr (EPI == EPI_SCALE_MIN)
    pad = (a.s0 >= 0.0f) ? __builtin_inff() : -__builtin_inff();
  int dir_neg = 0;  // a channel of this thread keeps its window minimum
  for (int co = tid; co < a.ncb * G::COUT; co += G::NTHR) {
    const bool real = co < a.Cout;
    float bv = pad, pv = 0.0f;
    if (real) {
      bv = a.b[co];
      if constexpr (EPI == EPI_MUL_LRELU_GELU)
        pv = a.v0[co] * kGeluIn;  // (the folded form of mul_lrelu_gelu_erf)
      if constexpr (EPI == EPI_MUL_LRELU_GELU_TANH)
        pv = a.v0[co];
      if constexpr (gn_epilogue<EPI>())
        pv = ((a.v0[co] >= 0.0f) == (a.v2[co] >= 0.0f)) ? 1.0f : -1.0f;
    }
    s_bias[co] = bv;
    s_par[co] = pv;
    dir_neg |= pv < 0.0f;
  }
  // (made visible by the barrier at the top of the first item)
  // Pooling epilogues: whether every channel keeps its window maximum
  // (gamma*scale >= 0 throughout, the usual case); then the extrema need
  // no direction factor.
  bool all_max = false;
  if constexpr (gn_epilogue<EPI>())
    all_max = __builtin_amdgcn_readfirstlane(!__syncthreads_or(dir_neg)) != 0;
  // Windows of any size (k >= 3) are combined across the wavefronts of a
  // tile in this buffer, [channel of the block][window row][window column]
  // of the tile, before they are stored; it starts (and is left) at -inf.
  // A channel's windows take at most WINCH slots (k >= 3), its fixed stride.
  constexpr int WINCH = (G::TH / 3) * (G::TWC / 3);
  constexpr int WINBUF = EPI == EPI_GN_POOLKL ? G::COUT * WINCH : 1;
  static_assert((G::LDS_DWORDS + 2 * kMaxCout + WINBUF) * 4 <= 160 * 1024,
                "LDS budget exceeded");
  __shared__ float s_win[WINBUF];
  if constexpr (EPI == EPI_GN_POOLKL) {
    for (int i = tid; i < WINBUF; i += G::NTHR) s_win[i] = -__builtin_inff();
  }

  f32x16 acc[G::MT][G::NW];
  // running channel extremum of the min epilogues, per N-tile, carried from
  // one channel-block pass of a tile to the next
  float run[G::NW];
#pragma unroll
  for (int j = 0; j < G::NW; ++j) run[j] = 0.0f;

  // Deferred stores of the channel-min epilogues: a tile's epilogue parks
  // its NW/2 results per lane here, and they are issued from the middle of
  // the next item's MFMA loop.  Stores count in vmcnt, so storing them at
  // once would make the wait for the next stage at the item start also wait
  // for their completion.  A parked offset with bit 31 set is dropped, so
  // the flush is unconditional.  (The GroupNorm epilogue stores at once:
  // parking its results raised the register count past the budget.)
  constexpr bool DEFER = EPI == EPI_MIN_TANH2 || EPI == EPI_SCALE_MIN;
  constexpr bool IS_GN = gn_epilogue<EPI>();
  // per-group partials (groups of 4 channels) or per-channel partials
  constexpr bool GN_CH =
      EPI == EPI_GN_POOL_CH || EPI == EPI_GN_POOLK_CH || EPI == EPI_GN_POOLKL;
  constexpr int NPEND = (DEFER && G::NW > 1) ? G::NW / 2 : 1;
  constexpr uint32_t DROP = 0x80000000u;
  uint32_t pend_v[NPEND], pend_off[NPEND];
#pragma unroll
  for (int k = 0; k < NPEND; ++k) {
    pend_v[k] = 0u;
    pend_off[k] = DROP;
  }
  int pend_n = 0;  // the parked results' sample (buffer resources rebuilt
                   // at the flush: one register instead of eight)
  // this sample's slice of out (and of the GroupNorm partials), as the
  // epilogues address them
  auto out_rsrc = [&](int n) X3_INLINE {
    if constexpr (IS_GN)
      return make_rsrc(a.out + (size_t)n * a.Cout * a.Ph * a.Pw,
                       (uint32_t)(a.Cout * a.Ph * a.Pw * 4));
    else
      return make_rsrc(a.out + (size_t)n * a.Ho * a.Wo, (uint32_t)(a.Ho * a.Wo * 4));
  };
  auto part_rsrc = [&](int n) X3_INLINE {
    const int pps = a.n_rt * a.n_ct * G::NWAVE;
    const int rows = GN_CH ? a.Cout : a.groups;
    return make_rsrc(a.part + (size_t)n * rows * pps, (uint32_t)(rows * pps * 16));
  };
  // Pin the parked values where the epilogue computed them: left free, the
  // compiler may sink their computation to the flush in the next item and
  // keep the old accumulators alive across it.
  auto pin_parked = [&]() X3_INLINE {
#pragma unroll
    for (int k = 0; k < NPEND; ++k) {
      asm volatile("" : "+v"(pend_v[k]));
      asm volatile("" : "+v"(pend_off[k]));
    }
  };
  auto flush = [&]() X3_INLINE {
    if constexpr (DEFER) {
      const __amdgpu_buffer_rsrc_t o_rsrc = out_rsrc(pend_n);
#pragma unroll
      for (int k = 0; k < NPEND; ++k) {
        __builtin_amdgcn_raw_buffer_store_b32(pend_v[k], o_rsrc, pend_off[k],
                                              0, 0);
        pend_off[k] = DROP;
      }
    }
  };

  auto epilogue = [&](int t, int cb) X3_INLINE {
    // ---- epilogue for channel block cb of tile t ------------------------------
    const int co0 = cb * G::COUT;
    const int ct = t % a.n_ct;
    const int rt = (t / a.n_ct) % a.n_rt;
    const int n = t / (a.n_ct * a.n_rt);
    const int r_base = rt * a.thk + wm.row0;           // output row of j = 0
    const int c = ct * a.twk + wm.strip * 32 + l32;    // output column
    const bool col_ok = c < a.Wo;

    if constexpr (EPI == EPI_MIN_TANH2 || EPI == EPI_SCALE_MIN) {
      // Channel extremum per pixel: in-lane over the lane's 16*MT channels,
      // then across the two lane halves (which hold the other channels of
      // the same pixels).  Half 0 finishes pixel rows 0..NW/2-1 and half 1
      // rows NW/2..NW-1, so every lane evaluates and stores NW/2 results.
      static_assert(G::NW % 2 == 0 || G::NW == 1, "lane halves split the N-tiles");
      constexpr int HN = G::NW / 2;
      const bool use_max = (EPI == EPI_SCALE_MIN) && !(a.s0 >= 0.0f);
      float m[G::NW];
      // (one uniform branch around two compile-time reductions, rather than
      // a min, a max and a select per element)
      auto reduce = [&](auto maxc) X3_INLINE {
        constexpr bool MX = decltype(maxc)::value;
#pragma unroll
        for (int j = 0; j < G::NW; ++j) {
          float v = acc[0][j][0];
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              v = MX ? fmaxf(v, acc[mt][j][i]) : fminf(v, acc[mt][j][i]);
          m[j] = v;
        }
      };
      if (use_max)
        reduce(std::true_type{});
      else
        reduce(std::false_type{});
      if (a.ncb > 1) {  // (uniform) fold in the earlier blocks' extremum
        const bool first = cb == 0;
#pragma unroll
        for (int j = 0; j < G::NW; ++j) {
          const float r = use_max ? fmaxf(m[j], run[j]) : fminf(m[j], run[j]);
          m[j] = first ? m[j] : r;
          run[j] = m[j];
        }
        if (cb != a.ncb - 1) return;  // more channel blocks to come
      }
      auto finish = [&](float v) X3_INLINE {
        if constexpr (EPI == EPI_MIN_TANH2)
          return tanh_e2(tanh_e2(v));
        else
          return a.s0 * v;
      };
      if constexpr (G::NW == 1) {
        // one pixel row: both halves hold the full extremum after the
        // exchange, half 0 stores it
        const float recv = shfl_xor(m[0], 32);
        const float v = use_max ? fmaxf(m[0], recv) : fminf(m[0], recv);
        pend_v[0] = __builtin_bit_cast(uint32_t, finish(v));
        pend_off[0] = ((uint32_t)(r_base * a.Wo + c) << 2) |
                      ((uint32_t)!(col_ok && r_base < a.Ho && h == 0) << 31);
      }
#pragma unroll
      for (int jj = 0; jj < HN; ++jj) {
        const float keep = h ? m[jj + HN] : m[jj];
        const float recv = shfl_xor(h ? m[jj] : m[jj + HN], 32);
        const float v = use_max ? fmaxf(keep, recv) : fminf(keep, recv);
        const int r = r_base + jj + h * HN;
        // bounded store into this sample's output plane (parked for the
        // next item's loop); bit 31 drops it
        pend_v[jj] = __builtin_bit_cast(uint32_t, finish(v));
        pend_off[jj] = ((uint32_t)(r * a.Wo + c) << 2) |
                       ((uint32_t)!(col_ok && r < a.Ho) << 31);
      }
      pend_n = n;
      pin_parked();
    } else if constexpr (EPI == EPI_MUL_LRELU_GELU ||
                         EPI == EPI_MUL_LRELU_GELU_TANH || EPI == EPI_STORE) {
      const float slope = a.s0;
      // bounded stores into this sample's [Cout][Ho][Wo] block; an offset
      // with bit 31 set (pixel outside the output) is dropped
      // (NCHW: padded channels land past the end of the block and are
      // dropped; NHWC: they would land in the next pixel, so they get the
      // drop bit)
      const int HoWo = a.Ho * a.Wo;
      const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(
          a.out + (size_t)n * a.Cout * HoWo, (uint32_t)(a.Cout * HoWo * 4));
      uint32_t pix_off[G::NW], drop[G::NW];
#pragma unroll
      for (int j = 0; j < G::NW; ++j) {
        const int r = r_base + j;
        pix_off[j] = (uint32_t)(r * a.Wo + c) * (G::NHWC ? (uint32_t)a.Cout : 1u);
        drop[j] = (uint32_t)!(col_ok && r < a.Ho) << 31;
      }
      const bool neg_slope = slope < 0.0f;
      auto op = [&](float y, float mv) X3_INLINE {
        if constexpr (EPI == EPI_MUL_LRELU_GELU)
          y = mul_lrelu_gelu_erf(y, mv, slope, neg_slope);
        else if constexpr (EPI == EPI_MUL_LRELU_GELU_TANH)
          y = gelu_tanh(lrelu(y * mv, slope));
        return y;
      };
      if (G::NHWC && (a.flags & kOutVec4)) {
        // NHWC with 16-byte stores: accumulator elements 4q..4q+3 are 4
        // consecutive channels of one pixel (a multiple of 4, so with
        // Cout % 4 == 0 the 4 are real or padded together).  Pixel row by
        // pixel row: the 2*MT*4 stores of a row complete its pixels' lines
        // back to back (2.4 % faster than channel group by channel group).
#pragma unroll
        for (int j = 0; j < G::NW; ++j)
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int co = co0 + mt * 32 + 8 * q + 4 * h;
            const uint32_t pad = (uint32_t)(co >= a.Cout) << 31;
            const f32x4 mv = *reinterpret_cast<const f32x4*>(&s_par[co]);
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = __builtin_bit_cast(uint32_t, op(acc[mt][j][4 * q + e], mv[e]));
            const uint32_t off =
                ((pix_off[j] + (uint32_t)co) << 2) | drop[j] | pad;
            __builtin_amdgcn_raw_buffer_store_b128(v, o_rsrc, off, 0, 0);
          }
        return;
      }
      if constexpr (G::NHWC) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int co = co0 + 4 * h + mt * 32 + 8 * (i >> 2) + (i & 3);
            const float mv = s_par[co];
            const uint32_t co_off = (uint32_t)co | ((uint32_t)(co >= a.Cout) << 31);
#pragma unroll
            for (int j = 0; j < G::NW; ++j) {
              // (OR, not add: nothing can clear the drop bits)
              const uint32_t off =
                  ((co_off + pix_off[j]) << 2) | drop[j] | (co_off & 0x80000000u);
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(uint32_t, op(acc[mt][j][i], mv)), o_rsrc, off, 0, 0);
            }
          }
        return;
      }
      // NCHW: each store goes through a buffer resource based at the plane
      // of lane half 0's channel cb (scalar: built per channel, with the
      // records up to the end of the sample's block), so its offset is the
      // lane's part alone -- lane half h's 4 channels further, plus the
      // pixel -- computed once per tile: no vector instruction per store.
      // A dropped pixel has bit 31 set, past every record count; a padded
      // channel lies at or past its resource's end (lane half 1 at
      // 4 * HoWo floats on, below 2 GiB since the padded channels' planes
      // are), and a channel block wholly past Cout gets no records.
      uint32_t voff[G::NW];
#pragma unroll
      for (int j = 0; j < G::NW; ++j)
        voff[j] = drop[j] ? drop[j] : ((uint32_t)(4 * h) * (uint32_t)HoWo + pix_off[j]) << 2;
      float* const ob = a.out + (size_t)n * a.Cout * HoWo;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cb = co0 + mt * 32 + 8 * (i >> 2) + (i & 3);
          const int left = a.Cout - cb;  // channels from cb to the block's end
          const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(
              ob + (size_t)cb * HoWo, left > 0 ? (uint32_t)left * (uint32_t)HoWo * 4u : 0u);
          const float mv = s_par[cb + 4 * h];
#pragma unroll
          for (int j = 0; j < G::NW; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, op(acc[mt][j][i], mv)), c_rsrc, voff[j], 0, 0);
        }
    } else {  // the GroupNorm epilogues: wave tiles of 4 rows
      static_assert(G::NW == 4, "GroupNorm epilogues need 4-row wave tiles");
      // Stores go through raw buffer resources over this sample's slice of
      // `part` and `out` (out_rsrc, part_rsrc); a store that must not happen
      // gets bit 31 set in its offset (past num_records, dropped by the
      // hardware), so the epilogue has no exec-masked branches.  Padded
      // channels and groups land past the ends and are dropped.
      const int PP = a.Ph * a.Pw;
      const int pps = a.n_rt * a.n_ct * G::NWAVE;
      const __amdgpu_buffer_rsrc_t o_rsrc = out_rsrc(n);
      // (1) GroupNorm partials of this wave: per group, the count, the sum
      // and the sum of squared deviations from the wave's own group mean,
      // over the wave's valid pixels.  A group is 4 consecutive channels,
      // which is exactly accumulator elements 4q..4q+3 of one lane.  The
      // deviations are taken in one pass from a shift K, a conv value of
      // the same group (so |mean - K| is of the order of the spread):
      // S1 = sum(x - K), S2 = sum((x - K)^2), M2 = S2 - S1^2 / n.
      // valid rows: inside the image and inside the tile's thk rows (a
      // prefix of the wave's rows); valid columns likewise
      int nrow_ok = min(a.Ho - r_base, a.thk - wm.row0);
      nrow_ok = nrow_ok < 0 ? 0 : (nrow_ok > G::NW ? G::NW : nrow_ok);
      int ncol_ok = min(a.Wo - (ct * a.twk + wm.strip * 32), a.twk - wm.strip * 32);
      ncol_ok = ncol_ok < 0 ? 0 : (ncol_ok > 32 ? 32 : ncol_ok);
      const bool col_ok = l32 < ncol_ok;
      const int slot = (rt * a.n_ct + ct) * G::NWAVE + wave;
      if constexpr (!GN_CH) {
      static_assert(G::MT == 2, "8 groups per lane half");
      const float cnt = (float)(4 * nrow_ok * ncol_ok);
      const float inv_cnt = cnt > 0.0f ? 1.0f / cnt : 0.0f;
      // shift of group gi = mt*4 + q: its first channel at the half's
      // first pixel
      f32x8 kv;
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) kv[gi] = half_lane0(acc[gi >> 2][0][4 * (gi & 3)]);
      // in-lane sums over the lane's pixels: sv[2gi] = S1, sv[2gi+1] = S2
      f32x16 sv;
      auto lane_sums = [&](auto masked) X3_INLINE {
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
          const int mt = gi >> 2, q = gi & 3;
          float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
          for (int j = 0; j < G::NW; ++j) {
            const bool ok = col_ok && j < nrow_ok;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float d = acc[mt][j][4 * q + e] - kv[gi];
              if constexpr (decltype(masked)::value) d = ok ? d : 0.0f;
              s1 += d;
              s2 = fmaf(d, d, s2);
            }
          }
          sv[2 * gi] = s1;
          sv[2 * gi + 1] = s2;
        }
      };
      // (uniform) whole wave tiles need no masks; with all rows valid, a
      // lane's column is wholly valid or not, so its sums are dropped after
      // the fact (16 selects instead of one per accumulator element)
      if (nrow_ok == G::NW) {
        lane_sums(std::false_type{});
        if (ncol_ok != 32) {
#pragma unroll
          for (int k = 0; k < 16; ++k) sv[k] = col_ok ? sv[k] : 0.0f;
        }
      } else {
        lane_sums(std::true_type{});
      }
      // Sums over the 32 lanes of a half by a halving exchange: in each
      // step a lane keeps the half of its values selected by one lane bit,
      // adds the partner's copy of that half and hands over the other
      // half.  Bits 3, 2, 0, 1 (DPP partners l^8 by a row rotation, l^7 by
      // the half-row mirror, then the quad), and finally l^16 for the one
      // value left.  Lane bits (3, 2, 0) then name the group and bit 1
      // whether the lane holds S1 or S2.
      const bool b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1,
                 b3 = (lane >> 3) & 1;
      f32x8 r8 = b3 ? sv.hi : sv.lo;
      {
        const f32x8 give = b3 ? sv.lo : sv.hi;
#pragma unroll
        for (int k = 0; k < 8; ++k) r8[k] += dpp<DPP_ROW_ROR8>(give[k]);
      }
      f32x4 r4 = b2 ? r8.hi : r8.lo;
      {
        const f32x4 give = b2 ? r8.lo : r8.hi;
#pragma unroll
        for (int k = 0; k < 4; ++k) r4[k] += dpp<DPP_ROW_HALF_MIRROR>(give[k]);
      }
      f32x2 r2 = b0 ? r4.hi : r4.lo;
      {
        const f32x2 give = b0 ? r4.lo : r4.hi;
#pragma unroll
        for (int k = 0; k < 2; ++k) r2[k] += dpp<DPP_QUAD_XOR1>(give[k]);
      }
      float S = (b1 ? r2.y : r2.x) + dpp<DPP_QUAD_XOR2>(b1 ? r2.x : r2.y);
      S += swz_xor16(S);
      const float S1 = S, S2 = dpp<DPP_QUAD_XOR2>(S);  // (valid where !b1)
      const int gi = 4 * b3 + 2 * b2 + b0;
      const f32x4 k4 = b3 ? kv.hi : kv.lo;
      const f32x2 k2 = b2 ? k4.hi : k4.lo;
      const float K = b0 ? k2.y : k2.x;
      {
        // lanes with bits 1 and 4 clear store group
        // g = co0/4 + mt*8 + 2q + h of gi = mt*4 + q
        const int g = (co0 >> 2) + (gi >> 2) * 8 + 2 * (gi & 3) + h;
        const uint32_t off = ((uint32_t)(g * pps + slot) << 4) |
                             ((uint32_t)((lane & 0x12) != 0) << 31);
        const float4 v = make_float4(fmaf(K, cnt, S1),
                                     fmaxf(S2 - S1 * S1 * inv_cnt, 0.0f), cnt, 0.0f);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, v), part_rsrc(n), off, 0, 0);
      }
      } else {
      // (1') Per-channel partials (any group size; the finalize merges the
      // group's channels): count, sum and M2 of each channel over the
      // wave's valid pixels, again about a shift K, the channel's value at
      // the wave's first pixel.  In-lane over the rows, then across the 32
      // columns of a lane half, 8 accumulator elements at a time, by a
      // halving exchange: in each of 3 steps a lane keeps half of its
      // channel sums, adds the partner's matching half and hands over the
      // other half.  The partners are l^16, l^15, l^7 (swizzle, row mirror,
      // half-row mirror) and the keep decision is lane bit 4, 3, 2; two
      // quad steps (l^1, l^2) complete the sums.  Each quad ends with
      // element (l32 >> 2) & 7 of the 8, and its first lane stores it.
      const __amdgpu_buffer_rsrc_t p_rsrc = part_rsrc(n);
      const float cnt = (float)(nrow_ok * ncol_ok);
      const float inv_cnt = cnt > 0.0f ? 1.0f / cnt : 0.0f;
      const bool b4 = (l32 >> 4) & 1, b3 = (l32 >> 3) & 1, b2 = (l32 >> 2) & 1;
      const int e8 = (l32 >> 2) & 7;
      const uint32_t not_lead = (uint32_t)((l32 & 3) != 0) << 31;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          // (vector values, not arrays: selects between array elements
          // would be turned into loads from selected addresses, which
          // keeps the arrays in scratch memory)
          f32x8 s1, s2, kv;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int i = 8 * hs + k;
            const float K = half_lane0(acc[mt][0][i]);
            kv[k] = K;
            float u1 = 0.0f, u2 = 0.0f;
#pragma unroll
            for (int j = 0; j < G::NW; ++j) {
              const float d = (col_ok && j < nrow_ok) ? acc[mt][j][i] - K : 0.0f;
              u1 += d;
              u2 = fmaf(d, d, u2);
            }
            s1[k] = u1;
            s2[k] = u2;
          }
          // partner l^16, keep by bit 4
          f32x4 t1 = b4 ? s1.hi : s1.lo, t2 = b4 ? s2.hi : s2.lo;
          const f32x4 g1 = b4 ? s1.lo : s1.hi, g2 = b4 ? s2.lo : s2.hi;
          const f32x4 kv4 = b4 ? kv.hi : kv.lo;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            t1[k] += swz_xor16(g1[k]);
            t2[k] += swz_xor16(g2[k]);
          }
          // partner l^15, keep by bit 3
          f32x2 r1 = b3 ? t1.hi : t1.lo, r2 = b3 ? t2.hi : t2.lo;
          const f32x2 h1 = b3 ? t1.lo : t1.hi, h2 = b3 ? t2.lo : t2.hi;
          const f32x2 kv2 = b3 ? kv4.hi : kv4.lo;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            r1[k] += dpp<DPP_ROW_MIRROR>(h1[k]);
            r2[k] += dpp<DPP_ROW_MIRROR>(h2[k]);
          }
          // partner l^7, keep by bit 2; then the quad
          float S1 = (b2 ? r1.y : r1.x) + dpp<DPP_ROW_HALF_MIRROR>(b2 ? r1.x : r1.y);
          float S2 = (b2 ? r2.y : r2.x) + dpp<DPP_ROW_HALF_MIRROR>(b2 ? r2.x : r2.y);
          S1 += dpp<DPP_QUAD_XOR1>(S1);
          S2 += dpp<DPP_QUAD_XOR1>(S2);
          S1 += dpp<DPP_QUAD_XOR2>(S1);
          S2 += dpp<DPP_QUAD_XOR2>(S2);
          const float K = b2 ? kv2.y : kv2.x;
          // element i = 8*hs + e8 is channel 8*(i>>2) + 4h + (i&3) of block mt
          const int co =
              co0 + mt * 32 + 8 * (2 * hs + (e8 >> 2)) + 4 * h + (e8 & 3);
          const float4 v = make_float4(fmaf(K, cnt, S1),
                                       fmaxf(S2 - S1 * S1 * inv_cnt, 0.0f), cnt,
                                       0.0f);
          const uint32_t off = ((uint32_t)(co * pps + slot) << 4) | not_lead;
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, v), p_rsrc, off, 0, 0);
        }
      }
      if constexpr (!gn_generic_k<EPI>()) {
        // (the statistics are complete: keep the window code from being
      // interleaved with them, which would hold both phases' values at once)
      __builtin_amdgcn_sched_barrier(0);
      // (2) 4x4 window extrema.  The wave's 4 N-tiles are 4 consecutive
        // rows starting at a multiple of 4, and 4 consecutive lanes are 4
        // consecutive columns starting at a multiple of 4, so a window is
        // (4 rows in-lane) x (4 lanes of a quad).  Only the extremum that the
        // monotone GroupNorm-affine-scale map sends to the window maximum is
        // stored: the max where gamma*scale >= 0, else the min.  Both are
        // taken as a maximum of sg*y, sg = +-1 the channel's direction (exact:
        // negation is exact and min(y) = -max(-y)), so each value enters one
        // max chain.  Across the quad a halving exchange on lane bits 0 and 1
        // leaves channel 2*b0 + b1 of the 4-channel block in each lane.
        const int py = r_base >> 2;
        const int px = c >> 2;
        const uint32_t win_off = (uint32_t)(py * a.Pw + px);
        const uint32_t win_bad = (uint32_t)!(py < a.Ph && px < a.Pw) << 31;
        const bool q0 = lane & 1, q1 = (lane >> 1) & 1;
        const int e = 2 * q0 + q1;
        // SG: per-channel direction factors; without (all_max) the chains
        // take the raw values.  (one uniform branch around two compile-time
        // forms)
        auto extrema = [&](auto sgc) X3_INLINE {
          constexpr bool SG = decltype(sgc)::value;
  #pragma unroll
          for (int mt = 0; mt < G::MT; ++mt)
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cq = co0 + mt * 32 + 8 * q + 4 * h;  // first channel
              f32x4 sg = {1.0f, 1.0f, 1.0f, 1.0f};
              if constexpr (SG) sg = *reinterpret_cast<const f32x4*>(&s_par[cq]);
              f32x4 t;
  #pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) {
                float m = SG ? sg[e2] * acc[mt][0][4 * q + e2] : acc[mt][0][4 * q + e2];
  #pragma unroll
                for (int j = 1; j < G::NW; ++j)
                  m = vmax(m, SG ? sg[e2] * acc[mt][j][4 * q + e2] : acc[mt][j][4 * q + e2]);
                t[e2] = m;
              }
              f32x2 u = q0 ? t.hi : t.lo;
              {
                const f32x2 give = q0 ? t.lo : t.hi;
  #pragma unroll
                for (int k = 0; k < 2; ++k) u[k] = vmax(u[k], dpp<DPP_QUAD_XOR1>(give[k]));
              }
              const float r = vmax(q1 ? u.y : u.x, dpp<DPP_QUAD_XOR2>(q1 ? u.x : u.y));
              float v = r;
              if constexpr (SG) {
                const f32x2 s2 = q0 ? sg.hi : sg.lo;
                v = (q1 ? s2.y : s2.x) * r;
              }
              const int co = cq + e;
              // NCHW: channel planes (padded channels fall past the end);
              // NHWC: channels innermost (padded channels get the drop bit)
              const uint32_t off =
                  G::NHWC ? ((win_off * (uint32_t)a.Cout + (uint32_t)co) << 2) |
                                win_bad | ((uint32_t)(co >= a.Cout) << 31)
                          : (((uint32_t)co * PP + win_off) << 2) | win_bad;
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v),
                                                    o_rsrc, off, 0, 0);
            }
        };
        if (all_max)
          extrema(std::false_type{});
        else
          extrema(std::true_type{});
      } else {
        // (2') Windows of any size k.  A tile's origin is a multiple of k
        // on both axes and it covers thk x twk outputs, both multiples of
        // k, so no window leaves its tile; a window whose row pk*py is past
        // Ph (or column past Pw) is an incomplete floor-mode window and is
        // dropped, and every conv output inside a kept window is inside
        // the image.  As for 4x4 windows, only the extremum that the
        // monotone GroupNorm-affine-scale map sends to the maximum is kept,
        // as a maximum of sg*y.
        const int pk = a.pk;
        const __amdgpu_buffer_rsrc_t o_rsrc = out_rsrc(n);
        // NCHW: channel planes; NHWC: channels innermost (padded channels
        // get the drop bit)
        auto win_store = [&](int co, int py, int px, bool ok, float v) X3_INLINE {
          const uint32_t bad = (uint32_t)!ok << 31;
          const uint32_t off =
              G::NHWC ? (((uint32_t)(py * a.Pw + px) * (uint32_t)a.Cout + (uint32_t)co) << 2) |
                            bad | ((uint32_t)(co >= a.Cout) << 31)
                      : (((uint32_t)co * PP + (uint32_t)(py * a.Pw + px)) << 2) | bad;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), o_rsrc,
                                                off, 0, 0);
        };
        if (EPI != EPI_GN_POOLKL && pk == 1) {
          // every conv output is its own window
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int co = co0 + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
#pragma unroll
              for (int j = 0; j < G::NW; ++j)
                win_store(co, r_base + j, c, col_ok && j < nrow_ok, acc[mt][j][i]);
            }
        } else if constexpr (EPI != EPI_GN_POOLKL) {
          // k = 2: a window is 2 rows in-lane (the wave's rows start at a multiple
          // of 4) x 2 adjacent lanes (columns start at a multiple of 32):
          // the pair's halving exchange leaves window row 2*(r_base/2) + b0
          // in lane half b0 = lane bit 0
          const bool b0 = lane & 1;
          const int py = (r_base >> 1) + b0, px = c >> 1;
          const bool wok = py < a.Ph && px < a.Pw;
          auto pairs = [&](auto sgc) X3_INLINE {
            constexpr bool SG = decltype(sgc)::value;
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int co = co0 + mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                const float sg = SG ? s_par[co] : 1.0f;
                const float t0 = vmax(sg * acc[mt][0][i], sg * acc[mt][1][i]);
                const float t1 = vmax(sg * acc[mt][2][i], sg * acc[mt][3][i]);
                const float r = vmax(b0 ? t1 : t0, dpp<DPP_QUAD_XOR1>(b0 ? t0 : t1));
                win_store(co, py, px, wok, SG ? sg * r : r);
              }
          };
          if (all_max)
            pairs(std::false_type{});
          else
            pairs(std::true_type{});
        } else {
          // k >= 3: windows cross wavefronts.  Each wave folds its rows of
          // a window in-lane (its 4 rows meet at most 2 window rows when k
          // >= 3) and merges the result into the tile's window buffer with
          // an LDS float maximum; lanes of one window column meet at the
          // same address.  After a workgroup barrier all threads store the
          // buffer and reset it to -inf.  (The next write to the buffer
          // comes after the next item's barrier.)
          const int nwx = a.twk / pk, nwy = a.thk / pk, nwin = nwx * nwy;
          const int wy0 = wm.row0 / pk;
          const int split = (wy0 + 1) * pk - wm.row0;  // rows j < split: wy0
          const int jlim = a.thk - wm.row0;             // rows j < jlim: in the tile
          const int cl = wm.strip * 32 + l32;           // column in the tile
          const bool lok = cl < a.twk;
          const int wx = lok ? cl / pk : 0;
          const int offA = min(wy0, nwy - 1) * nwx + wx;
          const int offB = min(wy0 + 1, nwy - 1) * nwx + wx;
          constexpr float NEG = -__builtin_inff();
          auto fold = [&](auto sgc) X3_INLINE {
            constexpr bool SG = decltype(sgc)::value;
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int chl = mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
                const float sg = SG ? s_par[co0 + chl] : 1.0f;
                float mA = NEG, mB = NEG;
#pragma unroll
                for (int j = 0; j < G::NW; ++j) {
                  const float v = SG ? sg * acc[mt][j][i] : acc[mt][j][i];
                  mA = (j < jlim && j < split) ? vmax(mA, v) : mA;
                  mB = (j < jlim && j >= split) ? vmax(mB, v) : mB;
                }
                // (constant channel stride: the offset is an immediate)
                float* w = s_win + chl * WINCH;
                __hip_atomic_fetch_max(w + offA, lok ? mA : NEG, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_max(w + offB, lok ? mB : NEG, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
              }
          };
          if (all_max)
            fold(std::false_type{});
          else
            fold(std::true_type{});
          __syncthreads();
          const int py0 = rt * a.thk / pk, px0 = ct * a.twk / pk;
          // (exact: the fractional parts sit at least 0.5 / nwin away from
          // an integer, far above the rounding of these small products)
          const float rnw = 1.0f / (float)nwin, rnx = 1.0f / (float)nwx;
          for (int idx = tid; idx < G::COUT * nwin; idx += G::NTHR) {
            const int chl = (int)(((float)idx + 0.5f) * rnw);
            const int wv = idx - chl * nwin;
            const int wy = (int)(((float)wv + 0.5f) * rnx);
            const int wxi = wv - wy * nwx;
            float v = s_win[chl * WINCH + wv];
            s_win[chl * WINCH + wv] = NEG;
            const int co = co0 + chl, py = py0 + wy, px = px0 + wxi;
            if (!all_max) v *= s_par[co];
            win_store(co, py, px, py < a.Ph && px < a.Pw, v);
          }
        }
      }
    }
  };

  // ---- one item: wait for its stage, prefetch the next item into the other
  // stage from inside the MFMA loop, multiply, and finish the tile ----------
  auto run_item = [&](auto bufc, int item, Pos& pos) X3_INLINE {
    constexpr int BUF = decltype(bufc)::value;
    X3_LDS float* cur = BUF ? (X3_LDS float*)lds1 : (X3_LDS float*)lds0;
    X3_LDS float* nxt = BUF ? (X3_LDS float*)lds0 : (X3_LDS float*)lds1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // the next item, or on the last item this item again (its data are
    // in bounds; the reload is never used)
    const bool has_next = item + 1 < nitems;
    const Pos np = advance(pos);
    Pos pp;
    pp.tl = has_next ? np.tl : pos.tl;
    pp.cb = has_next ? np.cb : pos.cb;
    pp.chunk = has_next ? np.chunk : pos.chunk;
    const Lim nl = lim_of(item_of(pp));
    int zz;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zz));

    const int cb = pos.cb, chunk = pos.chunk;
    const int t = vb + pos.tl * G_;

    // One resident K chunk (RC == 1; the host guarantees one chunk and one
    // channel block): every item starts a tile, and the first k-step's
    // MFMAs take the bias as their C operand (no accumulator moves).
    constexpr bool BIAS_C = G::RC == 1;
    f32x16 binit[BIAS_C ? G::MT : 1];
    if constexpr (BIAS_C) {
      const X3_LDS float* sb = (const X3_LDS float*)s_bias;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          binit[mt][i] = sb[mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3)];
    } else if (chunk == 0) {
      // accumulators start at the bias
      const X3_LDS float* sb = (const X3_LDS float*)s_bias + cb * G::COUT;
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float bv = sb[mt * 32 + 8 * (i >> 2) + 4 * h + (i & 3)];
#pragma unroll
          for (int j = 0; j < G::NW; ++j) acc[mt][j][i] = bv;
        }
    }

    // NH4: the lane's pixel for tap column kw, in the slot that holds its
    // half's channels (the slot order swaps every 8 columns)
    const X3_LDS float* xsk[3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
      xsk[kw] = cur + (wm.row0 * G::XCOLS + wm.strip * 32 + l32 + kw) * 8 +
                4 * (h ^ (((l32 + kw) >> 3) & 1));
    const X3_LDS float* xs =
        G::NH4    ? xsk[0]
        : G::NHWC ? cur + (wm.row0 * G::XCOLS + wm.strip * 32 + l32) * G::CCP + h
        : G::KO   ? cur + h * (G::CC / 2) * G::CS + wm.row0 * G::XP +
                        wm.strip * 32 + l32
                  : cur + h * G::CS + wm.row0 * G::XP + wm.strip * 32 + l32;
    // (a weight row holds K index ci*9 + tap, or with PW channel 4h + e of
    // tap t at dword 36h + 4t + e; lane half h starts at channel CC/2 * h
    // for KO and NH4, which is dword 36h = KS*h either way)
    const X3_LDS float* ws =
        (G::RESW ? (const X3_LDS float*)ldsw + chunk * G::WBUF
                 : cur + G::XBUF) + l32 * G::WP + h * (G::X4 ? G::KS : 9);
    // Software pipeline over the k-steps of the chunk: step s issues the LDS
    // fragment reads of step s+1, its share of the next item's staging
    // loads, then its MFMAs; a scheduling fence keeps that order, so each
    // MFMA's operands were requested a full step (MT*NW MFMAs) earlier.
    // KO and PW read the weights of 4 k-steps at once, a group ahead; NH4
    // reads the input values of the 4 k-steps of a tap at once, a tap ahead.
    float av[2][G::MT], bv[2][G::NW];
    constexpr bool A4 = G::KO || PW;  // weights of 4 k-steps in one read
    f32x4 a4[2][A4 ? G::MT : 1];
    f32x4 b4[2][G::NH4 ? G::NW : 1];
    auto load_b4 = [&](int tap, f32x4 (&Bq)[G::NH4 ? G::NW : 1]) X3_INLINE {
      const int kh = tap / 3, kw = tap % 3;
#pragma unroll
      for (int j = 0; j < (G::NH4 ? G::NW : 1); ++j)
        Bq[j] = *reinterpret_cast<const X3_LDS f32x4*>(xsk[kw] + (j + kh) * G::XCOLS * 8);
    };
    auto load_a4 = [&](int g, f32x4 (&A)[A4 ? G::MT : 1]) X3_INLINE {
#pragma unroll
      for (int mt = 0; mt < (A4 ? G::MT : 1); ++mt)
        A[mt] = *reinterpret_cast<const X3_LDS f32x4*>(ws + mt * 32 * G::WP +
                                                       4 * g);
    };
    auto load_frag = [&](int s, float (&A)[G::MT], float (&Bv)[G::NW]) X3_INLINE {
      if constexpr (G::NH4) {
        // k-step s: tap s/4, channel 4h + s%4 (K index (4h + s%4)*9 + tap);
        // with PW its weights come with the group's ds_read_b128
        if constexpr (!PW) {
          const int tap = s / 4, cq = s % 4;
#pragma unroll
          for (int mt = 0; mt < G::MT; ++mt)
            A[mt] = ws[mt * 32 * G::WP + cq * 9 + tap];
        }
        (void)A;
        (void)Bv;
      } else if constexpr (G::KO) {
        const int ci = s / 9, tap = s % 9, kh = tap / 3, kw = tap % 3;
#pragma unroll
        for (int j = 0; j < G::NW; ++j)
          Bv[j] = xs[ci * G::CS + (j + kh) * G::XP + kw];
      } else {
        const int tap = s / (G::CC / 2);
        const int cp = s % (G::CC / 2);
        const int kh = tap / 3, kw = tap % 3;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
          A[mt] = ws[mt * 32 * G::WP + cp * 18 + tap];
#pragma unroll
        for (int j = 0; j < G::NW; ++j)
          Bv[j] = G::NHWC ? xs[((j + kh) * G::XCOLS + kw) * G::CCP + 2 * cp]
                          : xs[2 * cp * G::CS + (j + kh) * G::XP + kw];
      }
    };
    if constexpr (A4) load_a4(0, a4[0]);
    if constexpr (G::NH4) load_b4(0, b4[0]);
    load_frag(0, av[0], bv[0]);
#pragma unroll
    for (int s = 0; s < G::KS; ++s) {
      if constexpr (A4) {
        if (s % 4 == 0 && s / 4 + 1 < G::KS / 4)
          load_a4(s / 4 + 1, a4[(s / 4 + 1) & 1]);
      }
      if constexpr (G::NH4) {
        if (s % 4 == 0 && s / 4 + 1 < G::KS / 4)
          load_b4(s / 4 + 1, b4[(s / 4 + 1) & 1]);
      }
      if (s + 1 < G::KS) load_frag(s + 1, av[(s + 1) & 1], bv[(s + 1) & 1]);
      // (unconditional: on the last item this reloads the current item's
      // data into the idle stage, which keeps the step free of branches)
      if (s < KS_ISSUE) {
#pragma unroll
        for (int u = 0; u < BPS; ++u)
          if (s * BPS + u < NB_W) issue(nl, nxt, s * BPS + u, zz);
      }
      // the previous tile's parked epilogue stores, once the staging loads
      // are out
      if (s == KS_ISSUE) flush();
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int j = 0; j < G::NW; ++j)
          acc[mt][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
              A4 ? a4[(s / 4) & 1][mt][s % 4] : av[s & 1][mt],
              G::NH4 ? b4[(s / 4) & 1][G::NH4 ? j : 0][s % 4] : bv[s & 1][j],
              (BIAS_C && s == 0) ? binit[BIAS_C ? mt : 0] : acc[mt][j], 0, 0, 0);
      // Issue order inside the step: each MFMA (64 cycles in the matrix
      // core) is followed by a slice of this wave's other work -- LDS
      // fragment reads, staging address arithmetic, one staging load -- so
      // that work issues while the MFMA runs instead of between MFMA bursts.
#pragma unroll
      for (int k = 0; k < G::MT * G::NW; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);  // SALU
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    if (chunk == a.nchunk - 1) epilogue(t, cb);
    pos = np;
  };

  Pos pos;
  pos.tl = 0;
  pos.cb = 0;
  pos.chunk = 0;
  if (nitems > 0) {
    const Lim l0 = lim_of(item_of(pos));
#pragma unroll
    for (int i = 0; i < NB_W; ++i) issue(l0, (X3_LDS float*)lds0, i, 0);
    if constexpr (G::RESW) {
      // the resident weight tiles, once: chunk c's K columns into slot c
      // (one channel block, so co0 = 0)
#pragma unroll
      for (int c = 0; c < G::RC; ++c) {
        if (c < a.nchunk) {
          Lim lc = l0;
          lc.wbase = c * G::CC * 9;
          if constexpr (PRE)
            lc.wr = make_rsrc(a.w + lc.wbase, (w_total - (uint32_t)lc.wbase) * 4u);
          const int kl = 9 * (a.Cin - c * G::CC);
          lc.kk_lim = kl < G::KC ? kl : G::KC;
          lc.wslot = c;
#pragma unroll
          for (int i = G::NBI; i < G::NBI + NBWK; ++i)
            issue(lc, (X3_LDS float*)lds0, i, 0);
        }
      }
    }
  }
#pragma unroll 1
  for (int item = 0; item < nitems; item += 2) {
    run_item(std::integral_constant<int, 0>{}, item, pos);
    if (item + 1 < nitems)
      run_item(std::integral_constant<int, 1>{}, item + 1, pos);
  }
  flush();  // the last tile's parked stores
  // the last item's (unused) prefetch must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// GroupNorm finalize: merge the partials of one (sample, group) in double,
// then normalize, apply the affine and the per-channel scale, and clamp, in
// place on the pooled extrema written by conv3x3_igemm_kernel<...,
// EPI_GN_POOL or EPI_GN_POOL_CH>.  The group's partials are `pps`
// consecutive float4 (per-wave partials of the group, or of each of its
// channels in turn).
struct GnFinArgs {
  const float4* part;
  const float* gamma;
  const float* beta;
  const float* scale;
  float* out;
  int groups, cpg;   // groups, channels per group
  int C;             // channels (NHWC finalize: the channel stride of out)
  int nchunk;        // NHWC finalize: workgroups per sample
  int pps;           // partials per (sample, group)
  int plane;         // Ph * Pw
  float eps, lo, hi;
  double count;      // elements per group: cpg * Ho * Wo
};

// A DPP lane permutation of a double (each 32-bit half moved by one DPP
// move; the controls used stay inside a row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF,
                                                             0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL,
                                                             0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Sum over the 64 lanes of a wavefront in double, the same value in every
// lane, in a fixed order: DPP steps inside each row of 16 lanes (the two
// quad swaps, then rotations of the row by 4 and by 8 lanes) leave each
// row's sum in its first lane, and the four row sums are read out and
// added.  (Vector-unit lane moves of a few cycles each, where a shuffle
// through the LDS crossbar waits for a round trip per step.)
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<DPP_QUAD_XOR1>(v);
  v += dpp_d<DPP_QUAD_XOR2>(v);
  v += dpp_d<DPP_ROW_ROR4>(v);
  v += dpp_d<DPP_ROW_ROR8>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

// Sum of a double over the workgroup (wavefront sums, then LDS); every
// thread gets the total.  `red` holds one slot per wavefront.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum_d(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

// One workgroup of NT threads per (sample, group).  The group's cpg pooled
// channel planes are one contiguous block of cpg*plane floats in `out`;
// with up to 4 channels and VEC (block 16-byte aligned) it is moved as
// float4, larger groups go channel by channel.
//
// Merge: every partial k holds (sum_k, M2_k, n_k) over its pixels, with
// M2_k taken about its own mean.  With N = sum n_k (known: channels x Ho x
// Wo), mean = sum_k sum_k / N and M2 = sum_k [M2_k + n_k (sum_k/n_k -
// mean)^2] (the parallel-variance combination of Chan, Golub and LeVeque),
// accumulated in double.
// Group statistics from the partials p[0..pps) (p0 = p[threadIdx.x], or
// zeros past pps, already loaded by the caller): mean and 1/sqrt(var+eps).
template <int NT>
__device__ __forceinline__ void gn_group_stats(const GnFinArgs& a,
                                               const float4* p, float4 p0,
                                               double* red0, double* red1,
                                               float& mu, float& rstd) {
  const int tid = threadIdx.x;
  double sum = (double)p0.x;
  for (int k = tid + NT; k < a.pps; k += NT) sum += (double)p[k].x;
  const double mean = block_sum<NT>(sum, red0) / a.count;
  double m2 = 0.0;
  if (p0.z > 0.0f) {
    const double d = (double)p0.x / (double)p0.z - mean;
    m2 = (double)p0.y + (double)p0.z * d * d;
  }
  for (int k = tid + NT; k < a.pps; k += NT) {
    const float4 v = p[k];
    if (v.z > 0.0f) {
      const double d = (double)v.x / (double)v.z - mean;
      m2 += (double)v.y + (double)v.z * d * d;
    }
  }
  m2 = block_sum<NT>(m2, red1);
  mu = (float)mean;
  rstd = (float)(1.0 / sqrt(m2 / a.count + (double)a.eps));
}

template <int NT, bool VEC>
__global__ void __launch_bounds__(NT) gn_finalize_kernel(const GnFinArgs a) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole wavefronts");
  __shared__ double red0[NT / 64], red1[NT / 64];
  const int ng = blockIdx.x;  // n * groups + g
  const int g = ng % a.groups;
  const int tid = threadIdx.x;
  const int total = a.cpg * a.plane;  // floats in the block
  float* o = a.out + (size_t)ng * total;
  const int nvec = VEC ? total / 4 : total;
  const float4* p = a.part + (size_t)ng * a.pps;

  const float4 p0 = tid < a.pps ? p[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  // this thread's first block element, requested now so that its latency
  // hides behind the statistics merge below
  float4 first = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid < nvec) {
    if constexpr (VEC)
      first = reinterpret_cast<const float4*>(o)[tid];
    else
      first.x = o[tid];
  }
  float mu, rstd;
  gn_group_stats<NT>(a, p, p0, red0, red1, mu, rstd);

  // z = ((v - mu) * rstd * gamma + beta) * scale = (v - mu) * A + Bc, with
  // A = rstd*gamma*scale and Bc = beta*scale per channel; monotone in v
  // with the sign of gamma*scale, as the pooling pass assumed.
  const int c0 = g * a.cpg;
  const float lo = a.lo, hi = a.hi;
  if (a.cpg > 4) {
    // any group size: channel by channel
    for (int c = 0; c < a.cpg; ++c) {
      const float A = rstd * a.gamma[c0 + c] * a.scale[c0 + c];
      const float Bc = a.beta[c0 + c] * a.scale[c0 + c];
      float* oc = o + (size_t)c * a.plane;
      for (int k = tid; k < a.plane; k += NT)
        oc[k] = fminf(fmaxf(fmaf(oc[k] - mu, A, Bc), lo), hi);
    }
    return;
  }
  // Up to 4 channels: per-channel constants as plain scalars, selected per
  // element (an indexed array or struct here ends up in LDS or scratch
  // memory).
  const int c1 = c0 + (a.cpg > 1), c2 = c0 + 2 * (a.cpg > 2),
            c3 = c0 + 3 * (a.cpg > 3);
  const float A0 = rstd * a.gamma[c0] * a.scale[c0];
  const float A1 = rstd * a.gamma[c1] * a.scale[c1];
  const float A2 = rstd * a.gamma[c2] * a.scale[c2];
  const float A3 = rstd * a.gamma[c3] * a.scale[c3];
  const float B0 = a.beta[c0] * a.scale[c0];
  const float B1 = a.beta[c1] * a.scale[c1];
  const float B2 = a.beta[c2] * a.scale[c2];
  const float B3 = a.beta[c3] * a.scale[c3];
  const int p1 = a.plane, p2 = 2 * a.plane, p3 = 3 * a.plane;
#define X3_GN_OUT(v, e)                                                     \
  fminf(fmaxf(fmaf((v) - mu,                                                \
                   (e) < p1 ? A0 : ((e) < p2 ? A1 : ((e) < p3 ? A2 : A3)), \
                   (e) < p1 ? B0 : ((e) < p2 ? B1 : ((e) < p3 ? B2 : B3))), \
              lo),                                                          \
        hi)
  if constexpr (VEC) {
    constexpr int PT = 4;
    if (nvec <= PT * NT) {
      // (uniform) at most PT float4 per thread: the thread's others are
      // requested together now, after the merge (before it they would
      // queue ahead of the partials that the merge waits for); an element
      // past the block gets bit 31 in its offset and reads as zero
      const __amdgpu_buffer_rsrc_t orr = make_rsrc(o, (uint32_t)nvec * 16u);
      float4 v[PT];
      v[0] = first;
#pragma unroll
      for (int r = 1; r < PT; ++r) {
        const uint32_t k = (uint32_t)(tid + r * NT);
        v[r] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(
                        orr, (k << 4) | ((uint32_t)(k >= (uint32_t)nvec) << 31), 0, 0));
      }
#pragma unroll
      for (int r = 0; r < PT; ++r) {
        const int k = tid + r * NT;
        if (k >= nvec) break;
        const int e = 4 * k;
        float4 w;
        w.x = X3_GN_OUT(v[r].x, e);
        w.y = X3_GN_OUT(v[r].y, e + 1);
        w.z = X3_GN_OUT(v[r].z, e + 2);
        w.w = X3_GN_OUT(v[r].w, e + 3);
        reinterpret_cast<float4*>(o)[k] = w;
      }
      return;
    }
  }
  for (int k = tid; k < nvec; k += NT) {
    if constexpr (VEC) {
      const float4 v =
          k == tid ? first : reinterpret_cast<const float4*>(o)[k];
      const int e = 4 * k;
      float4 r;
      r.x = X3_GN_OUT(v.x, e);
      r.y = X3_GN_OUT(v.y, e + 1);
      r.z = X3_GN_OUT(v.z, e + 2);
      r.w = X3_GN_OUT(v.w, e + 3);
      reinterpret_cast<float4*>(o)[k] = r;
    } else {
      const float v = k == tid ? first.x : o[k];
      o[k] = X3_GN_OUT(v, k);
    }
  }
#undef X3_GN_OUT
}

// The finalize for pooled extrema stored NHWC, out [B][Ph][Pw][C]: the
// channels of one pooled position are contiguous, so a workgroup takes a
// contiguous chunk of one sample's [plane][C] block (all groups) and moves
// it with 16-byte accesses (VEC: C % 4 == 0, out 16-byte aligned), after
// merging the statistics of every group of the sample (one wavefront per
// group at a time; the partials are few and L2-resident) into per-channel
// constants in LDS.
// When a wavefront has at most four groups of at most 128 partials and 64
// channels (the usual case), it requests its partials (two per lane and
// group) and its lanes' channel parameters first, then the thread's share
// of the chunk, and merges while the chunk is in flight: the merge waits
// only for what was issued ahead of the chunk.  (Requesting the chunk ahead of the partials was measured
// slower: the merge then waits behind those loads.)  Otherwise the
// partials are read in a loop after the chunk has been requested.
// The merge is one pass over the partials in double: with s_k = sum_k,
// N = sum n_k, mean = sum s_k / N and
//   M2 = sum_k M2_k + sum_k n_k (s_k/n_k - mean)^2
//      = sum_k (M2_k + s_k^2 / n_k) - (sum s_k)^2 / N,
// the same sum as the pairwise (Chan) combination, reordered so that each
// partial is read once.

constexpr int kFinNhwcThreads = 1024;
constexpr int kFinNhwcPerThread = 8;  // float4 (or floats) per thread

template <int NT, bool VEC>
__global__ void __launch_bounds__(NT) gn_finalize_nhwc_kernel(const GnFinArgs a) {
  __shared__ __attribute__((aligned(16))) float s_mu[kMaxCout];
  __shared__ __attribute__((aligned(16))) float s_A[kMaxCout];
  __shared__ __attribute__((aligned(16))) float s_B[kMaxCout];
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x / a.nchunk, chunk = blockIdx.x - n * a.nchunk;
  float* o = a.out + (size_t)n * a.plane * a.C;
  const int total = a.plane * a.C;
  const int span = NT * kFinNhwcPerThread;
  const int nel = VEC ? total / 4 : total;
  const int beg = chunk * span;
  const int end = min(beg + span, nel);
  const float4* pn = a.part + (size_t)n * a.groups * a.pps;

  // Loads through raw buffer resources: an element that must not be read
  // gets bit 31 set in its offset (past num_records, read as zero), so the
  // loads need no branches.
  // (uniform) the wavefront's partials, and its lanes' channel parameters
  // (lane l: channel l of the group), fit in registers
  constexpr int GPW = 4;  // groups per wavefront held in registers
  const bool held = a.groups <= GPW * NWV && a.pps <= 128 && a.cpg <= 64;
  float4 pv[GPW][2];
  float gam[GPW], bet[GPW], sca[GPW];
  if (held) {
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(pn, (uint32_t)(a.groups * a.pps) * 16u);
    const uint32_t cbytes = (uint32_t)(a.groups * a.cpg) * 4u;
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(a.gamma, cbytes);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(a.beta, cbytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scale, cbytes);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = wave + gi * NWV;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int k = lane + 64 * r;
        const uint32_t off = ((uint32_t)(g * a.pps + k) << 4) |
                             ((uint32_t)!(g < a.groups && k < a.pps) << 31);
        pv[gi][r] = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
      }
      const uint32_t coff = ((uint32_t)(g * a.cpg + lane) << 2) |
                            ((uint32_t)!(g < a.groups && lane < a.cpg) << 31);
      gam[gi] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(gr, coff, 0, 0));
      bet[gi] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(br, coff, 0, 0));
      sca[gi] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, coff, 0, 0));
    }
  }
  // this thread's share of the chunk
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(o, (uint32_t)total * 4u);
  float4 v4[VEC ? kFinNhwcPerThread : 1];
  float v1[VEC ? 1 : kFinNhwcPerThread];
#pragma unroll
  for (int r = 0; r < kFinNhwcPerThread; ++r) {
    const int k = beg + tid + r * NT;
    const uint32_t bad = (uint32_t)(k >= end) << 31;
    if constexpr (VEC)
      v4[r] = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(orr, ((uint32_t)k << 4) | bad, 0, 0));
    else
      v1[r] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(orr, ((uint32_t)k << 2) | bad, 0, 0));
  }

  // group g's mean and 1/sigma from the wavefront's sums
  auto stats = [&](double sum, double sq, float& mu, float& rstd) {
    sum = wave_sum_d(sum);
    sq = wave_sum_d(sq);
    const double mean = sum / a.count;
    const double m2 = fmax(sq - sum * mean, 0.0);
    mu = (float)mean;
    rstd = (float)(1.0 / sqrt(m2 / a.count + (double)a.eps));
  };
  auto add = [](const float4 v, double& sum, double& sq) {
    if (v.z > 0.0f) {
      sum += (double)v.x;
      sq += (double)v.y + (double)v.x * (double)v.x / (double)v.z;
    }
  };
  if (held) {
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int g = wave + gi * NWV;
      if (g < a.groups) {
        double sum = 0.0, sq = 0.0;
        add(pv[gi][0], sum, sq);
        add(pv[gi][1], sum, sq);
        float mu, rstd;
        stats(sum, sq, mu, rstd);
        if (lane < a.cpg) {
          const int c = g * a.cpg + lane;
          s_mu[c] = mu;
          s_A[c] = rstd * gam[gi] * sca[gi];
          s_B[c] = bet[gi] * sca[gi];
        }
      }
    }
  } else {
    for (int g = wave; g < a.groups; g += NWV) {
      const float4* p = pn + (size_t)g * a.pps;
      double sum = 0.0, sq = 0.0;
      for (int k = lane; k < a.pps; k += 64) add(p[k], sum, sq);
      float mu, rstd;
      stats(sum, sq, mu, rstd);
      for (int c = g * a.cpg + lane; c < (g + 1) * a.cpg; c += 64) {
        s_mu[c] = mu;
        s_A[c] = rstd * a.gamma[c] * a.scale[c];
        s_B[c] = a.beta[c] * a.scale[c];
      }
    }
  }
  __syncthreads();
  if constexpr (VEC) {
    // a float4 holds 4 consecutive channels c..c+3 (C % 4 == 0, so c is a
    // multiple of 4 and their constants are one 16-byte LDS read each); a
    // thread's next float4 lies 4*NT floats on, step channels further
    // (mod C): with C dividing 4*NT (C = 64, 128, ...) the channels stay
    // and the constants are read once
    const int step = (4 * NT) % a.C;
    int c = (4 * (beg + tid)) % a.C;
    float4 mu, A, Bc;
    auto fetch = [&] {
      mu = *reinterpret_cast<const float4*>(&s_mu[c]);
      A = *reinterpret_cast<const float4*>(&s_A[c]);
      Bc = *reinterpret_cast<const float4*>(&s_B[c]);
    };
    fetch();
#pragma unroll
    for (int r = 0; r < kFinNhwcPerThread; ++r) {
      if (r > 0 && step != 0) {
        c += step;
        c -= c >= a.C ? a.C : 0;
        fetch();
      }
      const int k = beg + tid + r * NT;
      if (k >= end) continue;
      float4 v = v4[r];
      v.x = fminf(fmaxf(fmaf(v.x - mu.x, A.x, Bc.x), a.lo), a.hi);
      v.y = fminf(fmaxf(fmaf(v.y - mu.y, A.y, Bc.y), a.lo), a.hi);
      v.z = fminf(fmaxf(fmaf(v.z - mu.z, A.z, Bc.z), a.lo), a.hi);
      v.w = fminf(fmaxf(fmaf(v.w - mu.w, A.w, Bc.w), a.lo), a.hi);
      reinterpret_cast<float4*>(o)[k] = v;
    }
  } else {
#pragma unroll
    for (int r = 0; r < kFinNhwcPerThread; ++r) {
      const int k = beg + tid + r * NT;
      if (k >= end) continue;
      const int c = k % a.C;
      o[k] = fminf(fmaxf(fmaf(v1[r] - s_mu[c], s_A[c], s_B[c]), a.lo), a.hi);
    }
  }
}

}  // namespace x3
