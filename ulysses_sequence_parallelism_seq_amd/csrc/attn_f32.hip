// fp32 attention: the exactness path (small shapes, fp32 inputs).
//
// Plain fp32 arithmetic, one wavefront per output row, no matrix cores: a
// lane computes the full dot product for one key (or query) of a 64-wide
// chunk, the wave reduces max/sum across lanes, and the output row is spread
// over the lanes (d/64 values each). The softmax is the online form
// (running max and sum per row), exact up to fp32 rounding.
//
// Forward: S = Q K^T / sqrt(d) over the allowed keys, O = softmax(S) V,
// lse = ln sum exp(S). Backward: D = rowsum(dO * O), P = exp(S - lse),
// dS = P (dO V^T - D), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO.
// Allowed keys: same document (cu_seqlens) and, when causal, key <= query.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Document [s, e) holding token t (largest k with cu[k] <= t; empty documents skipped).
__device__ __forceinline__ void doc_of(const int* cu, int ndoc, int N, int t, int& s, int& e) {
  if (!cu) {
    s = 0;
    e = N;
    return;
  }
  int lo = 0, hi = ndoc;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  s = cu[lo];
  e = cu[lo + 1];
}

template <int D>
__device__ __forceinline__ float dot_row(const float* a, const float* b) {
  float acc = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; ++c) acc = fmaf(a[c], b[c], acc);
  return acc;
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void fwd_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, float* __restrict__ o,
                                                       float* __restrict__ lse, const int* __restrict__ cu,
                                                       int ndoc, int N, int Hl, int units, int causal,
                                                       float scale) {
  constexpr int J = D / 64;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long long)units * N) return;  // whole wave leaves; no barriers below
  const int unit = (int)(row / N), t = (int)(row % N);
  const int g = unit / Hl, h = unit % Hl;
  int s, e;
  doc_of(cu, ndoc, N, t, s, e);
  const size_t rs = (size_t)Hl * D;
  const size_t base = ((size_t)g * N * Hl + h) * D;
  const float* qrow = q + base + (size_t)t * rs;
  const int kend = causal ? t + 1 : e;

  float oc[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) oc[jj] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j0 = s; j0 < kend; j0 += 64) {
    const int j = j0 + lane;
    float sc = -INFINITY;
    if (j < kend) sc = dot_row<D>(qrow, k + base + (size_t)j * rs) * scale;
    const float mn = fmaxf(m, wave_max(sc));
    const float alpha = expf(m - mn);
    const float p = (j < kend) ? expf(sc - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int jj = 0; jj < J; ++jj) oc[jj] *= alpha;
    const int cnt = min(64, kend - j0);
    for (int x = 0; x < cnt; ++x) {
      const float px = __shfl(p, x, 64);
      const float* vr = v + base + (size_t)(j0 + x) * rs;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) oc[jj] = fmaf(px, vr[lane + 64 * jj], oc[jj]);
    }
    m = mn;
  }
  float* orow = o + base + (size_t)t * rs;
  const float inv = 1.f / l;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) orow[lane + 64 * jj] = oc[jj] * inv;
  if (lane == 0) lse[(size_t)unit * N + t] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void delta_f32(const float* __restrict__ o,
                                                         const float* __restrict__ dout,
                                                         float* __restrict__ delta, int N, int Hl,
                                                         int units) {
  constexpr int J = D / 64;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long long)units * N) return;
  const int unit = (int)(row / N), t = (int)(row % N);
  const int g = unit / Hl, h = unit % Hl;
  const size_t off = ((size_t)g * N * Hl + h) * D + (size_t)t * Hl * D;
  float acc = 0.f;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) acc = fmaf(o[off + lane + 64 * jj], dout[off + lane + 64 * jj], acc);
  acc = wave_sum(acc);
  if (lane == 0) delta[(size_t)unit * N + t] = acc;
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void dq_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v,
                                                      const float* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      const float* __restrict__ delta,
                                                      float* __restrict__ dq, const int* __restrict__ cu,
                                                      int ndoc, int N, int Hl, int units, int causal,
                                                      float scale) {
  constexpr int J = D / 64;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long long)units * N) return;
  const int unit = (int)(row / N), t = (int)(row % N);
  const int g = unit / Hl, h = unit % Hl;
  int s, e;
  doc_of(cu, ndoc, N, t, s, e);
  const size_t rs = (size_t)Hl * D;
  const size_t base = ((size_t)g * N * Hl + h) * D;
  const float* qrow = q + base + (size_t)t * rs;
  const float* dorow = dout + base + (size_t)t * rs;
  const float lse_t = lse[(size_t)unit * N + t];
  const float d_t = delta[(size_t)unit * N + t];
  const int kend = causal ? t + 1 : e;
  float acc[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) acc[jj] = 0.f;
  for (int j0 = s; j0 < kend; j0 += 64) {
    const int j = j0 + lane;
    float ds = 0.f;
    if (j < kend) {
      const float p = expf(dot_row<D>(qrow, k + base + (size_t)j * rs) * scale - lse_t);
      const float dp = dot_row<D>(dorow, v + base + (size_t)j * rs);
      ds = p * (dp - d_t);
    }
    const int cnt = min(64, kend - j0);
    for (int x = 0; x < cnt; ++x) {
      const float dsx = __shfl(ds, x, 64);
      const float* kr = k + base + (size_t)(j0 + x) * rs;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) acc[jj] = fmaf(dsx, kr[lane + 64 * jj], acc[jj]);
    }
  }
  float* out = dq + base + (size_t)t * rs;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) out[lane + 64 * jj] = acc[jj] * scale;
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void dkdv_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        const float* __restrict__ dout,
                                                        const float* __restrict__ lse,
                                                        const float* __restrict__ delta,
                                                        float* __restrict__ dk, float* __restrict__ dv,
                                                        const int* __restrict__ cu, int ndoc, int N, int Hl,
                                                        int units, int causal, float scale) {
  constexpr int J = D / 64;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (long long)units * N) return;
  const int unit = (int)(row / N), j = (int)(row % N);
  const int g = unit / Hl, h = unit % Hl;
  int s, e;
  doc_of(cu, ndoc, N, j, s, e);
  const size_t rs = (size_t)Hl * D;
  const size_t base = ((size_t)g * N * Hl + h) * D;
  const float* krow = k + base + (size_t)j * rs;
  const float* vrow = v + base + (size_t)j * rs;
  const float* lse_u = lse + (size_t)unit * N;
  const float* delta_u = delta + (size_t)unit * N;
  const int qbeg = causal ? j : s;
  float ak[J], av[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) ak[jj] = av[jj] = 0.f;
  for (int i0 = qbeg; i0 < e; i0 += 64) {
    const int i = i0 + lane;
    float p = 0.f, ds = 0.f;
    if (i < e) {
      p = expf(dot_row<D>(q + base + (size_t)i * rs, krow) * scale - lse_u[i]);
      const float dp = dot_row<D>(dout + base + (size_t)i * rs, vrow);
      ds = p * (dp - delta_u[i]);
    }
    const int cnt = min(64, e - i0);
    for (int x = 0; x < cnt; ++x) {
      const float px = __shfl(p, x, 64);
      const float dsx = __shfl(ds, x, 64);
      const float* qr = q + base + (size_t)(i0 + x) * rs;
      const float* dr = dout + base + (size_t)(i0 + x) * rs;
#pragma unroll
      for (int jj = 0; jj < J; ++jj) {
        av[jj] = fmaf(px, dr[lane + 64 * jj], av[jj]);
        ak[jj] = fmaf(dsx, qr[lane + 64 * jj], ak[jj]);
      }
    }
  }
  float* ko = dk + base + (size_t)j * rs;
  float* vo = dv + base + (size_t)j * rs;
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    ko[lane + 64 * jj] = ak[jj] * scale;
    vo[lane + 64 * jj] = av[jj];
  }
}

unsigned row_blocks(const uly_host::AttnGeom& a) {
  const long long rows = (long long)a.G * a.Hl * a.N;
  return (unsigned)((rows + kWaves - 1) / kWaves);
}

}  // namespace

namespace uly_host {

int launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                        const AttnGeom& a, void* stream) {
  const float scale = 1.0f / sqrtf((float)a.d);
  const int units = a.G * a.Hl;
  hipStream_t st = (hipStream_t)stream;
  if (a.d == 64)
    hipLaunchKernelGGL(fwd_f32<64>, dim3(row_blocks(a)), dim3(64 * kWaves), 0, st, q, k, v, o, lse, a.cu,
                       a.ndoc, a.N, a.Hl, units, a.causal, scale);
  else
    hipLaunchKernelGGL(fwd_f32<128>, dim3(row_blocks(a)), dim3(64 * kWaves), 0, st, q, k, v, o, lse, a.cu,
                       a.ndoc, a.N, a.Hl, units, a.causal, scale);
  return launch_status();
}

int launch_attn_bwd_prepare_f32(const float* o, const float* dout, float* delta, const AttnGeom& a,
                                void* stream) {
  const int units = a.G * a.Hl;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(row_blocks(a)), block(64 * kWaves);
  if (a.d == 64)
    hipLaunchKernelGGL(delta_f32<64>, grid, block, 0, st, o, dout, delta, a.N, a.Hl, units);
  else
    hipLaunchKernelGGL(delta_f32<128>, grid, block, 0, st, o, dout, delta, a.N, a.Hl, units);
  return launch_status();
}

int launch_attn_bwd_main_f32(const float* q, const float* k, const float* v, const float* dout,
                             const float* lse, float* dq, float* dk, float* dv, const float* delta,
                             const AttnGeom& a, void* stream) {
  const float scale = 1.0f / sqrtf((float)a.d);
  const int units = a.G * a.Hl;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(row_blocks(a)), block(64 * kWaves);
  if (a.d == 64) {
    hipLaunchKernelGGL(dq_f32<64>, grid, block, 0, st, q, k, v, dout, lse, delta, dq, a.cu, a.ndoc, a.N,
                       a.Hl, units, a.causal, scale);
    hipLaunchKernelGGL(dkdv_f32<64>, grid, block, 0, st, q, k, v, dout, lse, delta, dk, dv, a.cu, a.ndoc,
                       a.N, a.Hl, units, a.causal, scale);
  } else {
    hipLaunchKernelGGL(dq_f32<128>, grid, block, 0, st, q, k, v, dout, lse, delta, dq, a.cu, a.ndoc, a.N,
                       a.Hl, units, a.causal, scale);
    hipLaunchKernelGGL(dkdv_f32<128>, grid, block, 0, st, q, k, v, dout, lse, delta, dk, dv, a.cu,
                       a.ndoc, a.N, a.Hl, units, a.causal, scale);
  }
  return launch_status();
}

int launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                        const float* dout, const float* lse, float* dq, float* dk, float* dv,
                        float* delta, const AttnGeom& a, void* stream) {
  const int rc = launch_attn_bwd_prepare_f32(o, dout, delta, a, stream);
  if (rc != ULY_OK) return rc;
  return launch_attn_bwd_main_f32(q, k, v, dout, lse, dq, dk, dv, delta, a, stream);
}

}  // namespace uly_host
