// epilogue_kernels.hpp -- the four epilogues as standalone kernels over a
// stored conv output y [B][C][H][W] (NCHW, fp32).  They serve the split
// path: a caller's own convolution output, the unfused comparison against
// the fused kernels, and pooling windows that the fused GroupNorm epilogue
// does not cover.  Each reads y once, with 16-byte loads where the layout
// allows, and is bound by HBM bandwidth (the GELU form by its arithmetic
// nearly as much).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epi_math.hpp"

namespace x3 {

constexpr int kEpiThreads = 256;

// Streaming (non-temporal) 16-byte loads and stores: y is read once and the
// outputs are not read back by these kernels, so neither should displace
// cache lines that other traffic reuses.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const nt_f32x4 v =
      __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float4 r, float4* p) {
  nt_f32x4 v;
  v.x = r.x;
  v.y = r.y;
  v.z = r.z;
  v.w = r.w;
  __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
}

// ---------------------------------------------------------------------------
// Channel extremum: out[n][p] = tanh(tanh(min_c y[n][c][p])), or
// min_c(scale * y[n][c][p]) = scale * (scale >= 0 ? min_c y : max_c y).
enum ChanMode : int { CHAN_MIN_TANH2 = 0, CHAN_SCALE_MIN = 1 };

struct ChanArgs {
  const float* y;
  float* out;
  int C;
  int64_t P;        // pixels per channel plane (H * W)
  int64_t nchunk;   // blocks per sample
  float scale;
};

template <int MODE>
__device__ __forceinline__ float chan_finish(float m, float scale) {
  if constexpr (MODE == CHAN_MIN_TANH2)
    return tanh_e2(tanh_e2(m));
  else
    return scale * m;
}

// One thread per pixel, or per 4 pixels with VEC (P % 4 == 0 and both
// buffers 16-byte aligned).  The channel loop keeps 8 (VEC) or 4 loads in
// flight.
template <int MODE, bool VEC>
__global__ void __launch_bounds__(kEpiThreads) chan_extremum_kernel(const ChanArgs a) {
  const int64_t n = blockIdx.x / a.nchunk;
  const int64_t chunk = blockIdx.x - n * a.nchunk;
  const float* yn = a.y + n * a.C * a.P;
  float* on = a.out + n * a.P;
  const bool use_max = (MODE == CHAN_SCALE_MIN) && !(a.scale >= 0.0f);
  auto pick = [&](float u, float v) {
    return use_max ? fmaxf(u, v) : fminf(u, v);
  };
  if constexpr (VEC) {
    const int64_t q = chunk * kEpiThreads + threadIdx.x;  // float4 index
    const int64_t nq = a.P / 4;
    if (q >= nq) return;
    const float4* src = reinterpret_cast<const float4*>(yn) + q;
    float4 m = src[0];
    int c = 1;
    for (; c + 7 < a.C; c += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_stream(src + (c + u) * nq);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        m.x = pick(m.x, v[u].x);
        m.y = pick(m.y, v[u].y);
        m.z = pick(m.z, v[u].z);
        m.w = pick(m.w, v[u].w);
      }
    }
    for (; c < a.C; ++c) {
      const float4 v = src[c * nq];
      m.x = pick(m.x, v.x);
      m.y = pick(m.y, v.y);
      m.z = pick(m.z, v.z);
      m.w = pick(m.w, v.w);
    }
    float4 r;
    r.x = chan_finish<MODE>(m.x, a.scale);
    r.y = chan_finish<MODE>(m.y, a.scale);
    r.z = chan_finish<MODE>(m.z, a.scale);
    r.w = chan_finish<MODE>(m.w, a.scale);
    reinterpret_cast<float4*>(on)[q] = r;
  } else {
    const int64_t p = chunk * kEpiThreads + threadIdx.x;
    if (p >= a.P) return;
    const float* src = yn + p;
    float m = src[0];
    int c = 1;
    for (; c + 3 < a.C; c += 4)
      m = pick(pick(m, src[(c + 0) * a.P]),
               pick(pick(src[(c + 1) * a.P], src[(c + 2) * a.P]), src[(c + 3) * a.P]));
    for (; c < a.C; ++c) m = pick(m, src[c * a.P]);
    on[p] = chan_finish<MODE>(m, a.scale);
  }
}

// ---------------------------------------------------------------------------
// Elementwise: out = gelu(lrelu(y * mult[c], slope)), erf form (TANH false)
// or tanh form.  out may be y itself (each element is read, then written,
// by the same thread).
struct EwArgs {
  const float* y;
  const float* mult;
  float* out;
  int C;
  int64_t P;        // elements per channel plane
  int64_t nchunk;   // blocks per plane
  int64_t total4;   // flat form: float4 in the whole tensor
  float slope;
};

constexpr int kEwPerThread = 4;  // float4 (or floats) per thread

// m: the multiplier, times kGeluIn for the erf form (see mul_lrelu_gelu_erf)
template <bool TANH>
__device__ __forceinline__ float ew_op(float y, float m, float slope) {
  if constexpr (TANH) return gelu_tanh(lrelu(y * m, slope));
  else return mul_lrelu_gelu_erf(y, m, slope, slope < 0.0f);
}

template <bool TANH, bool VEC>
__global__ void __launch_bounds__(kEpiThreads) mul_lrelu_gelu_kernel(const EwArgs a) {
  const int64_t plane = blockIdx.x / a.nchunk;  // n * C + c
  const int64_t chunk = blockIdx.x - plane * a.nchunk;
  const float m = a.mult[plane % a.C] * (TANH ? 1.0f : kGeluIn);
  const float* src = a.y + plane * a.P;
  float* dst = a.out + plane * a.P;
  const int64_t first = chunk * (kEpiThreads * kEwPerThread) + threadIdx.x;
  if constexpr (VEC) {
    const int64_t nq = a.P / 4;
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4* d4 = reinterpret_cast<float4*>(dst);
    float4 v[kEwPerThread];
#pragma unroll
    for (int k = 0; k < kEwPerThread; ++k) {
      const int64_t q = first + k * kEpiThreads;
      if (q < nq) v[k] = ld_stream(s4 + q);
    }
#pragma unroll
    for (int k = 0; k < kEwPerThread; ++k) {
      const int64_t q = first + k * kEpiThreads;
      if (q < nq) {
        float4 r;
        r.x = ew_op<TANH>(v[k].x, m, a.slope);
        r.y = ew_op<TANH>(v[k].y, m, a.slope);
        r.z = ew_op<TANH>(v[k].z, m, a.slope);
        r.w = ew_op<TANH>(v[k].w, m, a.slope);
        st_stream(r, d4 + q);
      }
    }
  } else {
    float v[kEwPerThread];
#pragma unroll
    for (int k = 0; k < kEwPerThread; ++k) {
      const int64_t e = first + k * kEpiThreads;
      if (e < a.P) v[k] = src[e];
    }
#pragma unroll
    for (int k = 0; k < kEwPerThread; ++k) {
      const int64_t e = first + k * kEpiThreads;
      if (e < a.P) dst[e] = ew_op<TANH>(v[k], m, a.slope);
    }
  }
}

// The same operation over the tensor as one flat float4 array (P % 4 == 0,
// both buffers 16-byte aligned, P / 4 >= the block's span): block b takes
// the float4 [b*span, (b+1)*span), so every block is full (except the
// tensor's last) and starts on a 16 KB boundary; a float4 never straddles
// two planes and a block meets at most two, whose multipliers it reads
// once.  Measured 10 % faster than the per-plane blocks on [64,64,254,254]
// (whose last block in each plane is three-quarters full).
template <bool TANH>
__global__ void __launch_bounds__(kEpiThreads) mul_lrelu_gelu_flat4_kernel(const EwArgs a) {
  constexpr int SPAN = kEpiThreads * kEwPerThread;
  const int64_t per = a.P / 4;
  const int64_t b0 = (int64_t)blockIdx.x * SPAN;
  const int64_t plane0 = b0 / per;
  const int64_t qb = (plane0 + 1) * per;  // first float4 of the next plane
  const float k = TANH ? 1.0f : kGeluIn;
  const float m0 = a.mult[plane0 % a.C] * k;
  const float m1 = a.mult[(plane0 + 1) % a.C] * k;
  const float4* s4 = reinterpret_cast<const float4*>(a.y);
  float4* d4 = reinterpret_cast<float4*>(a.out);
  float4 v[kEwPerThread];
#pragma unroll
  for (int r = 0; r < kEwPerThread; ++r) {
    const int64_t q = b0 + threadIdx.x + r * kEpiThreads;
    if (q < a.total4) v[r] = ld_stream(s4 + q);
  }
#pragma unroll
  for (int r = 0; r < kEwPerThread; ++r) {
    const int64_t q = b0 + threadIdx.x + r * kEpiThreads;
    if (q < a.total4) {
      const float m = q < qb ? m0 : m1;
      float4 o;
      o.x = ew_op<TANH>(v[r].x, m, a.slope);
      o.y = ew_op<TANH>(v[r].y, m, a.slope);
      o.z = ew_op<TANH>(v[r].z, m, a.slope);
      o.w = ew_op<TANH>(v[r].w, m, a.slope);
      st_stream(o, d4 + q);
    }
  }
}

// ---------------------------------------------------------------------------
// GroupNorm -> per-channel scale -> MaxPool2d(k, stride k, floor) -> clamp
// on a stored y, in one read of y: this kernel, one workgroup per (sample,
// channel) plane, then the GroupNorm finalize of the fused path.
//
// The map z = (y - mean) * A + Bc (A = rstd*gamma*scale, Bc = beta*scale)
// is monotone in y with the sign of A, so the window maximum of z is z of
// the window maximum of y where gamma*scale >= 0 and of the window minimum
// otherwise.  The plane kernel walks the pooling windows: every element
// feeds the plane's statistics (sums of d = y - K and d^2 about K, the
// plane's first element, per thread in fp32 over its few dozen elements,
// then over the workgroup in double), and each window's raw extremum is
// parked in out.  The elements outside every window (the floor-mode
// remainder rows and columns) feed the statistics only.  The plane's
// (sum, M2, count) goes to part[n][c]; the finalize merges the cpg partials
// of a group and maps the parked extrema through z and the clamp.
struct GnPlaneArgs {
  const float* y;
  const float* gamma;
  const float* scale;
  float* out;    // [B][C][Ph][Pw] parked extrema
  float4* part;  // [B][C] plane partials
  int C, H, W, k, Ph, Pw;
};

// Quad permutation of a float (DPP quad_perm; 0xB1 swaps lanes 0<->1 and
// 2<->3 of each quad, 0x4E swaps 0<->2 and 1<->3).
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

template <int NT>
__device__ __forceinline__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) v += __shfl_xor(v, mask, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

// Lanes run along a row: each wavefront step ("unit") takes one row of
// windows and a span of 64/k*k consecutive columns (whole windows), so
// every load instruction reads consecutive floats and every element in a
// window is loaded exactly once.  The k rows of a window are reduced
// in-lane, then the k lanes of the window by shuffles (butterflies for
// k = 4, KT = 4; any k with KT = 0).
template <int KT>
__global__ void __launch_bounds__(kEpiThreads) gn_plane_kernel(const GnPlaneArgs a) {
  constexpr int NT = kEpiThreads, NWV = NT / 64;
  __shared__ double red0[NT / 64], red1[NT / 64];
  const int64_t nc = blockIdx.x;  // n * C + c
  const int c = (int)(nc % a.C);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // (the host keeps a plane below 2^31 floats: 32-bit indices)
  const int P = a.H * a.W, PP = a.Ph * a.Pw;
  const float* yb = a.y + nc * (int64_t)P;
  float* ob = a.out + nc * (int64_t)PP;
  const int k = KT ? KT : a.k;
  const bool keep_max = (a.gamma[c] >= 0.0f) == (a.scale[c] >= 0.0f);

  const float Kf = yb[0];
  float s1 = 0.0f, s2 = 0.0f;
  auto acc = [&](float v) {
    const float d = v - Kf;
    s1 += d;
    s2 = fmaf(d, d, s2);
  };
  // pass 1a: the windows.  Each step issues the loads of UNR units before
  // reducing any of them (one unit's loads alone would leave the
  // wavefront waiting on one round trip to memory per unit).
  const int span = (64 / k) * k;           // columns per unit
  const int cw = a.Pw * k, rh = a.Ph * k;  // window-covered columns / rows
  const int nsx = (cw + span - 1) / span;  // units per row of windows
  const int nunits = a.Ph * nsx;
  const int lead = lane - lane % k;        // first lane of this lane's window
  constexpr int UNR = KT == 4 ? 4 : 1;
  for (int u0 = wave; u0 < nunits; u0 += NWV * UNR) {
    float v[UNR][KT == 4 ? 4 : 1];
    int pyq[UNR], xq[UNR];
    bool okq[UNR];
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const int u = u0 + q * NWV;
      const int py = u / nsx;
      const int x = (u - py * nsx) * span + lane;
      pyq[q] = py;
      xq[q] = x;
      okq[q] = u < nunits && lane < span && x < cw;
      if constexpr (KT == 4) {
        // (a unit past the end, or a lane past the windows, addresses the
        // plane's first row instead, so no load can leave the plane)
        const float* src = yb + (okq[q] ? py * 4 * a.W + x : 0);
        // (unconditional loads from valid addresses: no branch separates
        // them, so all UNR*4 are in flight together.  Ordinary, not
        // streaming, loads: rows need not start on a cache line, and a line
        // shared by two units or rows should survive until both used it.)
#pragma unroll
        for (int dy = 0; dy < 4; ++dy)
          v[q][dy] = src[dy * a.W];
      }
    }
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const bool ok = okq[q];
      const int py = pyq[q], x = xq[q];
      float mx = -__builtin_inff(), mn = __builtin_inff();
      if constexpr (KT == 4) {
        float wmx = fmaxf(fmaxf(v[q][0], v[q][1]), fmaxf(v[q][2], v[q][3]));
        float wmn = fminf(fminf(v[q][0], v[q][1]), fminf(v[q][2], v[q][3]));
#pragma unroll
        for (int dy = 0; dy < 4; ++dy) {
          const float d = ok ? v[q][dy] - Kf : 0.0f;
          s1 += d;
          s2 = fmaf(d, d, s2);
        }
        mx = ok ? wmx : mx;
        mn = ok ? wmn : mn;
        // the 4 lanes of a window are a quad
        mx = fmaxf(mx, quad_swap<0xB1>(mx));
        mn = fminf(mn, quad_swap<0xB1>(mn));
        mx = fmaxf(mx, quad_swap<0x4E>(mx));
        mn = fminf(mn, quad_swap<0x4E>(mn));
      } else {
        const float* src = yb + (ok ? py * k * a.W + x : 0);
        for (int dy = 0; dy < k; ++dy) {
          if (ok) {
            const float w = src[dy * a.W];
            acc(w);
            mx = fmaxf(mx, w);
            mn = fminf(mn, w);
          }
        }
        const float m0 = mx, n0 = mn;
        for (int j = 1; j < k; ++j) {
          mx = fmaxf(mx, __shfl(m0, lead + j, 64));
          mn = fminf(mn, __shfl(n0, lead + j, 64));
        }
      }
      if (ok && lane == lead) ob[py * a.Pw + x / k] = keep_max ? mx : mn;
    }
  }
  // pass 1b: the remainder, the columns right of the last window (all
  // rows), then the rows below the last window; 4 loads in flight
  const int right = a.H * (a.W - cw), below = (a.H - rh) * cw;
  const int rem = right + below;
  for (int e0 = tid; e0 < rem; e0 += 4 * NT) {
    float w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i0 = e0 + q * NT;
      const int i = i0 < rem ? i0 : 0;  // (past the end: element 0 again)
      int row, col;
      if (i < right) {
        row = i / (a.W - cw);
        col = cw + (i - row * (a.W - cw));
      } else {
        const int j = i - right;
        row = rh + j / cw;
        col = j - (row - rh) * cw;
      }
      const float t = yb[row * a.W + col];
      w[q] = i0 < rem ? t : Kf;  // (Kf adds nothing)
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc(w[q]);
  }
  const double S1 = block_sum_d<NT>((double)s1, red0);
  const double S2 = block_sum_d<NT>((double)s2, red1);
  if (tid == 0) {
    const double n = (double)P;
    a.part[nc] = make_float4((float)(n * (double)Kf + S1),
                             (float)fmax(S2 - S1 * S1 / n, 0.0), (float)n, 0.0f);
  }
}

// The same operation for 4x4 windows and an even row length: lanes take 2
// adjacent columns each (8-byte loads), so one wavefront step covers 128
// columns of 4 rows -- a whole row of 126 floats in one load instruction
// -- and a window is 2 lanes.  Each step reads every column of its rows
// (the columns right of the last window feed only the statistics); the
// rows below the last window are read afterwards for the statistics.
// (a template only so that every translation unit may include it)
template <int K4 = 4>
__global__ void __launch_bounds__(kEpiThreads) gn_plane_k4w2_kernel(const GnPlaneArgs a) {
  constexpr int NT = kEpiThreads, NWV = NT / 64;
  __shared__ double red0[NT / 64], red1[NT / 64];
  const int64_t nc = blockIdx.x;  // n * C + c
  const int c = (int)(nc % a.C);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.H * a.W, PP = a.Ph * a.Pw;
  const float* yb = a.y + nc * (int64_t)P;
  float* ob = a.out + nc * (int64_t)PP;
  const bool keep_max = (a.gamma[c] >= 0.0f) == (a.scale[c] >= 0.0f);
  const float Kf = yb[0];
  float s1 = 0.0f, s2 = 0.0f;
  const int cw = a.Pw * 4, rh = a.Ph * 4;
  const int nsx = (a.W + 127) / 128;       // 128-column steps per row band
  const int nunits = a.Ph * nsx;
  constexpr int UNR = 4;
  for (int u0 = wave; u0 < nunits; u0 += NWV * UNR) {
    float2 v[UNR][4];
    int pyq[UNR], xq[UNR];
    bool okq[UNR];
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const int u = u0 + q * NWV;
      const int py = u / nsx;
      const int x = (u - py * nsx) * 128 + 2 * lane;  // this lane's first column
      pyq[q] = py;
      xq[q] = x;
      okq[q] = u < nunits && x < a.W;  // (W even: x + 1 < W too)
      // (a unit past the end, or a lane past the row, reads the plane's
      // first two columns instead: no load leaves the plane)
      const float* src = yb + (okq[q] ? py * 4 * a.W + x : 0);
#pragma unroll
      for (int dy = 0; dy < 4; ++dy)
        v[q][dy] = *reinterpret_cast<const float2*>(src + dy * a.W);
    }
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const bool ok = okq[q];
      float mx = -__builtin_inff(), mn = __builtin_inff();
#pragma unroll
      for (int dy = 0; dy < 4; ++dy) {
        const float d0 = ok ? v[q][dy].x - Kf : 0.0f;
        const float d1 = ok ? v[q][dy].y - Kf : 0.0f;
        s1 += d0 + d1;
        s2 = fmaf(d0, d0, fmaf(d1, d1, s2));
        mx = fmaxf(mx, fmaxf(v[q][dy].x, v[q][dy].y));
        mn = fminf(mn, fminf(v[q][dy].x, v[q][dy].y));
      }
      // the 2 lanes of a window are an even/odd pair
      mx = fmaxf(mx, quad_swap<0xB1>(mx));
      mn = fminf(mn, quad_swap<0xB1>(mn));
      const int x = xq[q];
      if (ok && (lane & 1) == 0 && x + 3 < cw)
        ob[pyq[q] * a.Pw + x / 4] = keep_max ? mx : mn;
    }
  }
  // the rows below the last window, for the statistics (8-byte pairs)
  const int half = a.W / 2;
  const int rem = (a.H - rh) * half;
  for (int e0 = tid; e0 < rem; e0 += 4 * NT) {
    float2 w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + q * NT < rem ? e0 + q * NT : 0;
      w[q] = *reinterpret_cast<const float2*>(yb + rh * a.W + 2 * e);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = e0 + q * NT < rem;
      const float d0 = ok ? w[q].x - Kf : 0.0f, d1 = ok ? w[q].y - Kf : 0.0f;
      s1 += d0 + d1;
      s2 = fmaf(d0, d0, fmaf(d1, d1, s2));
    }
  }
  const double S1 = block_sum_d<NT>((double)s1, red0);
  const double S2 = block_sum_d<NT>((double)s2, red1);
  if (tid == 0) {
    const double n = (double)P;
    a.part[nc] = make_float4((float)(n * (double)Kf + S1),
                             (float)fmax(S2 - S1 * S1 / n, 0.0), (float)n, 0.0f);
  }
}

// The whole GroupNorm epilogue in one kernel, one workgroup per (sample,
// group), for 4x4 windows, an even row length and a group whose pooled
// block (cpg * Ph * Pw floats) fits the dynamic LDS: wavefront w walks the
// group's planes w, w + NWV, ... as gn_plane_k4w2_kernel does (8-byte
// loads, 3 units in flight, within 64 registers for 8 wavefronts per SIMD)
// and parks each window's extremum in LDS instead
// of in out.  Each plane's (sum, M2) about its own first element is
// reduced over the wavefront in double; the group's mean and variance
// follow from the pairwise (Chan) combination of its planes; the parked
// extrema are then normalized, scaled and clamped on their way to out.  y
// is read once and out written once, with no workspace and no second
// kernel.
#define X3_EPI_INLINE __attribute__((always_inline))
constexpr int kGnGroupMaxCpg = 64;
constexpr int kGnGroupMaxLdsBytes = 48 * 1024;

struct GnGroupArgs {
  const float* y;
  const float* gamma;
  const float* beta;
  const float* scale;
  float* out;  // [B][C][Ph][Pw]
  int C, H, W, Ph, Pw, cpg;
  float eps, lo, hi;
};

// Sum over the 64 lanes of a wavefront, the same value in every lane, in
// a fixed order: DPP steps inside each row of 16 lanes (the two quad swaps,
// then rotations of the row by 4 and by 8 lanes) leave every lane with its
// row's sum, and the four row sums are read out and added.  (Lane
// permutations on the vector unit: a few cycles each, where a shuffle
// through the LDS crossbar waits for a round trip.)
__device__ __forceinline__ float wave_sum64_f(float v) {
  v += quad_swap<0xB1>(v);
  v += quad_swap<0x4E>(v);
  v += quad_swap<0x124>(v);  // row rotate right by 4
  v += quad_swap<0x128>(v);  // row rotate right by 8
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// (a template only so that every translation unit may include it)
template <int K4 = 4>
__global__ void __launch_bounds__(kEpiThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
gn_group_k4w2_kernel(const GnGroupArgs a) {
  constexpr int NT = kEpiThreads, NWV = NT / 64;
  // [cpg][Ph*Pw] parked extrema (16-byte aligned: read as float4 below)
  extern __shared__ __attribute__((aligned(16))) float s_ext[];
  __shared__ double s_ps[kGnGroupMaxCpg], s_pm[kGnGroupMaxCpg];
  __shared__ float s_A[kGnGroupMaxCpg], s_B[kGnGroupMaxCpg];
  __shared__ float s_mu;
  const int groups = a.C / a.cpg;
  const int n = blockIdx.x / groups, g = blockIdx.x - n * groups;
  const int c0 = g * a.cpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread p < cpg computes plane p's output map after the statistics:
  // its parameters are requested now, while the group streams in
  float gam = 0.0f, sca = 0.0f, bet = 0.0f;
  if (tid < a.cpg) {
    gam = a.gamma[c0 + tid];
    sca = a.scale[c0 + tid];
    bet = a.beta[c0 + tid];
  }
  const int P = a.H * a.W, PP = a.Ph * a.Pw;
  const int cw = a.Pw * 4, rh = a.Ph * 4;
  const int nsx = (a.W + 127) / 128;  // 128-column steps per row band
  const int nunits = a.Ph * nsx;
  for (int pl = wave; pl < a.cpg; pl += NWV) {
    const int c = c0 + pl;
    const float* yb = a.y + ((int64_t)n * a.C + c) * P;
    float* eb = s_ext + pl * PP;
    // (uniform per wavefront) the plane keeps its windows' maximum or
    // minimum: the direction the GroupNorm-affine-scale map preserves
    const bool keep_max = (a.gamma[c] >= 0.0f) == (a.scale[c] >= 0.0f);
    const float Kf = yb[0];
    float s1 = 0.0f, s2 = 0.0f;
    constexpr int UNR = 3;  // units in flight (4 would exceed 64 registers)
    // unit u: row band py, this lane's first column x (recomputed after
    // the loads rather than kept: registers bound the occupancy here)
    auto unit = [&](int u, int& py, int& x) X3_EPI_INLINE {
      py = u / nsx;
      x = (u - py * nsx) * 128 + 2 * lane;
      return u < nunits && x < a.W;  // (W even: x + 1 < W too)
    };
    // One compile-time direction per loop (one extremum chain per element
    // instead of a maximum and a minimum), and a lane's unit sums dropped
    // after the fact when the unit or its columns are not in the plane
    // (two selects per unit instead of one per element).
    auto stream = [&](auto maxc) X3_EPI_INLINE {
      constexpr bool MX = decltype(maxc)::value;
      for (int u0 = 0; u0 < nunits; u0 += UNR) {
        float2 v[UNR][4];
#pragma unroll
        for (int q = 0; q < UNR; ++q) {
          int py, x;
          const bool ok = unit(u0 + q, py, x);
          // (a unit past the end, or a lane past the row, reads the plane's
          // first two columns instead: no load leaves the plane)
          const float* src = yb + (ok ? py * 4 * a.W + x : 0);
#pragma unroll
          for (int dy = 0; dy < 4; ++dy)
            v[q][dy] = *reinterpret_cast<const float2*>(src + dy * a.W);
        }
#pragma unroll
        for (int q = 0; q < UNR; ++q) {
          int py, x;
          const bool ok = unit(u0 + q, py, x);
          float u1 = 0.0f, u2 = 0.0f;
          float m = MX ? -__builtin_inff() : __builtin_inff();
#pragma unroll
          for (int dy = 0; dy < 4; ++dy) {
            const float d0 = v[q][dy].x - Kf, d1 = v[q][dy].y - Kf;
            u1 += d0 + d1;
            u2 = fmaf(d0, d0, fmaf(d1, d1, u2));
            m = MX ? fmaxf(m, fmaxf(v[q][dy].x, v[q][dy].y))
                   : fminf(m, fminf(v[q][dy].x, v[q][dy].y));
          }
          s1 += ok ? u1 : 0.0f;
          s2 += ok ? u2 : 0.0f;
          // the 2 lanes of a window are an even/odd pair
          m = MX ? fmaxf(m, quad_swap<0xB1>(m)) : fminf(m, quad_swap<0xB1>(m));
          if (ok && (lane & 1) == 0 && x + 3 < cw) eb[py * a.Pw + x / 4] = m;
        }
      }
    };
    if (keep_max)
      stream(std::true_type{});
    else
      stream(std::false_type{});
    // the rows below the last window, for the statistics (8-byte pairs)
    const int half = a.W / 2;
    const int rem = (a.H - rh) * half;
    for (int e0 = lane; e0 < rem; e0 += 4 * 64) {
      float2 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + q * 64 < rem ? e0 + q * 64 : 0;
        w[q] = *reinterpret_cast<const float2*>(yb + rh * a.W + 2 * e);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = e0 + q * 64 < rem;
        const float d0 = ok ? w[q].x - Kf : 0.0f, d1 = ok ? w[q].y - Kf : 0.0f;
        s1 += d0 + d1;
        s2 = fmaf(d0, d0, fmaf(d1, d1, s2));
      }
    }
    // (the lane sums about Kf carry no large common offset, so their float
    // sum over the wavefront is good to a few ulp; the plane's (sum, M2)
    // are then formed in double)
    const double S1 = (double)wave_sum64_f(s1);
    const double S2 = (double)wave_sum64_f(s2);
    if (lane == 0) {
      const double np = (double)P;
      s_ps[pl] = np * (double)Kf + S1;        // the plane's sum
      s_pm[pl] = fmax(S2 - S1 * S1 / np, 0.0);  // its M2 about its mean
    }
  }
  __syncthreads();
  if (tid < a.cpg) {
    // Chan: M2 = sum_p [M2_p + P (mean_p - mean)^2], all planes of P
    // elements; each of these threads forms the same sums in the same order
    const double np = (double)P, total = np * a.cpg;
    double sum = 0.0;
    for (int p = 0; p < a.cpg; ++p) sum += s_ps[p];
    const double mean = sum / total;
    double m2 = 0.0;
    for (int p = 0; p < a.cpg; ++p) {
      const double dm = s_ps[p] / np - mean;
      m2 += s_pm[p] + np * dm * dm;
    }
    const float rstd = (float)(1.0 / sqrt(m2 / total + (double)a.eps));
    s_A[tid] = rstd * gam * sca;
    s_B[tid] = bet * sca;
    if (tid == 0) s_mu = (float)mean;
  }
  __syncthreads();
  const float mu = s_mu;
  // the group's output planes are one contiguous block of cpg * PP floats
  float* ob = a.out + ((int64_t)n * a.C + c0) * PP;
  const int tot = a.cpg * PP;
  if ((((uintptr_t)ob & 15u) | (uint32_t)(tot & 3)) == 0) {
    // 16-byte stores; an element's plane is idx / PP, taken as
    // (idx + 0.5) * (1 / PP) (exact: the block fits kGnGroupMaxLdsBytes,
    // so tot <= 12288 and the product's rounding stays far below its
    // distance 0.5 / PP to an integer)
    const float rpp = 1.0f / (float)PP;
    for (int k = tid; 4 * k < tot; k += NT) {
      const float4 e = *reinterpret_cast<const float4*>(s_ext + 4 * k);
      float r[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pl = (int)(((float)(4 * k + q) + 0.5f) * rpp);
        r[q] = fminf(fmaxf(fmaf(r[q] - mu, s_A[pl], s_B[pl]), a.lo), a.hi);
      }
      *reinterpret_cast<float4*>(ob + 4 * k) = make_float4(r[0], r[1], r[2], r[3]);
    }
  } else {
    for (int pl = 0; pl < a.cpg; ++pl) {
      const float A = s_A[pl], Bc = s_B[pl];
      for (int k = tid; k < PP; k += NT)
        ob[pl * PP + k] = fminf(fmaxf(fmaf(s_ext[pl * PP + k] - mu, A, Bc), a.lo), a.hi);
    }
  }
}


}  // namespace x3
