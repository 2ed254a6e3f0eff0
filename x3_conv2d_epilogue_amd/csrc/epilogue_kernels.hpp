// epilogue_kernels.hpp -- the four epilogues as standalone kernels over a
// stored conv output y [B][C][H][W] (NCHW, fp32).  They serve the split
// path: a caller's own convolution output, the unfused comparison against
// the fused kernels, and pooling windows that the fused GroupNorm epilogue
// does not cover.  All are bound by HBM bandwidth: y is read once (twice for
// GroupNorm: statistics, then the pooled normalization, the second read
// mostly from L2), with 16-byte loads where the layout allows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epi_math.hpp"

namespace x3 {

constexpr int kEpiThreads = 256;

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
    return tanhf(tanhf(m));
  else
    return scale * m;
}

// One thread per pixel, or per 4 pixels with VEC (P % 4 == 0 and both
// buffers 16-byte aligned).  The channel loop keeps 4 loads in flight.
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
    for (; c + 3 < a.C; c += 4) {
      const float4 v0 = src[(c + 0) * nq], v1 = src[(c + 1) * nq];
      const float4 v2 = src[(c + 2) * nq], v3 = src[(c + 3) * nq];
      m.x = pick(pick(m.x, v0.x), pick(pick(v1.x, v2.x), v3.x));
      m.y = pick(pick(m.y, v0.y), pick(pick(v1.y, v2.y), v3.y));
      m.z = pick(pick(m.z, v0.z), pick(pick(v1.z, v2.z), v3.z));
      m.w = pick(pick(m.w, v0.w), pick(pick(v1.w, v2.w), v3.w));
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
  float slope;
};

constexpr int kEwPerThread = 4;  // float4 (or floats) per thread

template <bool TANH>
__device__ __forceinline__ float ew_op(float y, float m, float slope) {
  const float v = lrelu(y * m, slope);
  return TANH ? gelu_tanh(v) : gelu_erf(v);
}

template <bool TANH, bool VEC>
__global__ void __launch_bounds__(kEpiThreads) mul_lrelu_gelu_kernel(const EwArgs a) {
  const int64_t plane = blockIdx.x / a.nchunk;  // n * C + c
  const int64_t chunk = blockIdx.x - plane * a.nchunk;
  const float m = a.mult[plane % a.C];
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
      if (q < nq) v[k] = s4[q];
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
        d4[q] = r;
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

// ---------------------------------------------------------------------------
// GroupNorm -> per-channel scale -> MaxPool2d(k, stride k, floor) -> clamp.
// One workgroup per (sample, group): the group's cpg channel planes are one
// contiguous block of y.  Pass 1: count-free shifted sums in double about
// K = the block's first element, giving mean = K + S1/N and
// M2 = S2 - S1^2/N (biased variance M2/N).  Pass 2: every pooled output of
// the group: the maximum over its k x k window of
// z = ((y - mean) * rstd * gamma + beta) * scale, clamped to [lo, hi].
struct GnPoolArgs {
  const float* y;
  const float* gamma;
  const float* beta;
  const float* scale;
  float* out;
  int groups, cpg;
  int H, W, k, Ph, Pw;
  float eps, lo, hi;
};

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

template <bool VEC>
__global__ void __launch_bounds__(kEpiThreads) gn_pool_kernel(const GnPoolArgs a) {
  constexpr int NT = kEpiThreads;
  __shared__ double red0[NT / 64], red1[NT / 64];
  const int64_t ng = blockIdx.x;  // n * groups + g
  const int g = (int)(ng % a.groups);
  const int tid = threadIdx.x;
  const int64_t P = (int64_t)a.H * a.W;
  const int64_t total = (int64_t)a.cpg * P;
  const float* yb = a.y + ng * total;

  const double K = (double)yb[0];
  double s1 = 0.0, s2 = 0.0;
  if constexpr (VEC) {
    const float4* y4 = reinterpret_cast<const float4*>(yb);
    for (int64_t q = tid; q < total / 4; q += NT) {
      const float4 v = y4[q];
      const double d0 = (double)v.x - K, d1 = (double)v.y - K;
      const double d2 = (double)v.z - K, d3 = (double)v.w - K;
      s1 += (d0 + d1) + (d2 + d3);
      s2 = fma(d0, d0, fma(d1, d1, fma(d2, d2, fma(d3, d3, s2))));
    }
  } else {
    for (int64_t i = tid; i < total; i += NT) {
      const double d = (double)yb[i] - K;
      s1 += d;
      s2 = fma(d, d, s2);
    }
  }
  const double S1 = block_sum_d<NT>(s1, red0);
  const double S2 = block_sum_d<NT>(s2, red1);
  const double N = (double)total;
  const double m2 = fmax(S2 - S1 * S1 / N, 0.0);
  const float mu = (float)(K + S1 / N);
  const float rstd = (float)(1.0 / sqrt(m2 / N + (double)a.eps));

  const int64_t PP = (int64_t)a.Ph * a.Pw;
  float* ob = a.out + ng * a.cpg * PP;
  const int c0 = g * a.cpg;
  for (int64_t o = tid; o < a.cpg * PP; o += NT) {
    const int c = (int)(o / PP);
    const int64_t r = o - c * PP;
    const int py = (int)(r / a.Pw), px = (int)(r - (int64_t)py * a.Pw);
    const float A = rstd * a.gamma[c0 + c] * a.scale[c0 + c];
    const float Bc = a.beta[c0 + c] * a.scale[c0 + c];
    const float* src = yb + c * P + (int64_t)py * a.k * a.W + (int64_t)px * a.k;
    float m = -__builtin_inff();
    for (int dy = 0; dy < a.k; ++dy)
      for (int dx = 0; dx < a.k; ++dx)
        m = fmaxf(m, fmaf(src[(int64_t)dy * a.W + dx] - mu, A, Bc));
    ob[o] = fminf(fmaxf(m, a.lo), a.hi);
  }
}

}  // namespace x3
