// Sequence-parallel loss aggregation over sp virtual ranks held on one device
// (jianying88 guide to DeepSpeed Ulysses in Transformers, section on the work
// Trainer does by itself, item 3): every rank's loss is the mean over its own
// counted tokens (labels other than the ignore index), the ranks' losses and
// counts are gathered, and the batch loss is sum_r loss_r * good_r /
// sum_r good_r over the ranks with good_r > 0. On a real SP group the gather is
// an all_gather of two numbers per rank; here the ranks' slices are stacked.
//
// Two launches, fixed order of every sum (bit-reproducible):
//   * partial kernel, grid (blocks per rank, sp): each thread walks its
//     rank's tokens four at a time (one 16-byte loss load, two 16-byte label
//     loads) when every rank's slice is 16-byte aligned, else one at a time,
//     keeps the counted ones in an fp64 sum and an int64 count, and the block
//     reduces them (wave shuffles, then LDS) to one partial;
//   * final kernel, one workgroup: rank r's partials summed in block order,
//     loss_r = sum / good_r (0 when good_r = 0), then the weighted mean over
//     ranks, summed in a fixed tree order.
// HBM-bound: 12 bytes read per token.

#include "common.h"

namespace {

constexpr int kLossThreads = 256;
constexpr int kTokPerThread = 16;  // per block pass: a block covers 4096 tokens
constexpr int kMaxBlocksPerRank = 256;

__device__ __forceinline__ void add_if(double& s, long long& c, float x, long long lab, long long ignore) {
  if (lab != ignore) {
    s += (double)x;
    c += 1;
  }
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// kVec: 4 tokens per load (each rank's slice 16-byte aligned); else one at a time
template <bool kVec>
__global__ __launch_bounds__(kLossThreads) void loss_partial_kernel(const float* __restrict__ token_loss,
                                                                    const long long* __restrict__ labels,
                                                                    double* __restrict__ psum,
                                                                    long long* __restrict__ pcnt, long long n,
                                                                    long long ignore) {
  __shared__ double ssum[kLossThreads / 64];
  __shared__ long long scnt[kLossThreads / 64];
  const int r = blockIdx.y;
  const float* tl = token_loss + (size_t)r * n;
  const long long* lb = labels + (size_t)r * n;
  double s = 0.0;
  long long c = 0;
  const long long stride = (long long)gridDim.x * kLossThreads;
  const long long first = (long long)blockIdx.x * kLossThreads + threadIdx.x;
  if constexpr (kVec) {
    // groups of 4 tokens (n % 4 == 0), dealt round-robin over the rank's threads
    for (long long gidx = first; gidx < n / 4; gidx += stride) {
      const float4 x = *reinterpret_cast<const float4*>(tl + 4 * gidx);
      const longlong2 l01 = *reinterpret_cast<const longlong2*>(lb + 4 * gidx);
      const longlong2 l23 = *reinterpret_cast<const longlong2*>(lb + 4 * gidx + 2);
      add_if(s, c, x.x, l01.x, ignore);
      add_if(s, c, x.y, l01.y, ignore);
      add_if(s, c, x.z, l23.x, ignore);
      add_if(s, c, x.w, l23.y, ignore);
    }
  } else {
    for (long long t = first; t < n; t += stride) add_if(s, c, tl[t], lb[t], ignore);
  }
  s = wave_sum(s);
  c = wave_sum(c);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ssum[w] = s;
    scnt[w] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ts = 0.0;
    long long tc = 0;
#pragma unroll
    for (int i = 0; i < kLossThreads / 64; ++i) {
      ts += ssum[i];
      tc += scnt[i];
    }
    psum[(size_t)r * gridDim.x + blockIdx.x] = ts;
    pcnt[(size_t)r * gridDim.x + blockIdx.x] = tc;
  }
}

// One workgroup; thread r handles rank r (sp <= kLossThreads * kRanksPerThread).
constexpr int kRanksPerThread = 16;
__global__ __launch_bounds__(kLossThreads) void loss_final_kernel(const double* __restrict__ psum,
                                                                  const long long* __restrict__ pcnt, int nblk,
                                                                  int sp, float* __restrict__ rank_loss,
                                                                  long long* __restrict__ good,
                                                                  float* __restrict__ loss) {
  __shared__ double wnum[kLossThreads / 64];
  __shared__ long long wden[kLossThreads / 64];
  double num = 0.0;
  long long den = 0;
  for (int j = 0; j < kRanksPerThread; ++j) {
    const int r = j * kLossThreads + threadIdx.x;
    if (r >= sp) break;
    double s = 0.0;
    long long c = 0;
    for (int b = 0; b < nblk; ++b) {
      s += psum[(size_t)r * nblk + b];
      c += pcnt[(size_t)r * nblk + b];
    }
    const double lr = c > 0 ? s / (double)c : 0.0;
    rank_loss[r] = (float)lr;
    good[r] = c;
    if (c > 0) {
      num += lr * (double)c;
      den += c;
    }
  }
  // fixed-order tree over the threads: butterfly within each wave, then the
  // four waves in order
  num = wave_sum(num);
  den = wave_sum(den);
  if ((threadIdx.x & 63) == 0) {
    wnum[threadIdx.x >> 6] = num;
    wden[threadIdx.x >> 6] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double tn = 0.0;
    long long td = 0;
#pragma unroll
    for (int i = 0; i < kLossThreads / 64; ++i) {
      tn += wnum[i];
      td += wden[i];
    }
    *loss = td > 0 ? (float)(tn / (double)td) : 0.f;
  }
}

int blocks_per_rank(long long n) {
  const long long per_block = (long long)kLossThreads * kTokPerThread;
  long long b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > kMaxBlocksPerRank) b = kMaxBlocksPerRank;
  return (int)b;
}

bool sizes_ok(int sp, int B, int Ns) {
  return sp > 0 && B > 0 && Ns > 0 && sp <= kLossThreads * kRanksPerThread && (long long)B * Ns < (1LL << 40);
}

}  // namespace

extern "C" size_t ulysses_sp_loss_workspace_bytes(int sp, int B, int Ns) {
  if (!sizes_ok(sp, B, Ns)) return 0;
  return (size_t)sp * blocks_per_rank((long long)B * Ns) * (sizeof(double) + sizeof(long long));
}

extern "C" int ulysses_sp_loss(const float* token_loss, const long long* labels, float* rank_loss,
                               long long* good_tokens, float* loss, void* workspace, size_t workspace_bytes, int sp,
                               int B, int Ns, int ignore_index, void* stream) {
  if (!token_loss || !labels || !rank_loss || !good_tokens || !loss) return ULY_EINVAL;
  if (!sizes_ok(sp, B, Ns)) return sp > kLossThreads * kRanksPerThread ? ULY_ESHAPE : ULY_EINVAL;
  const long long n = (long long)B * Ns;
  // 16-byte loads when every rank's slice starts 16-byte aligned
  const bool vec = n % 4 == 0 && ((uintptr_t)token_loss % 16) == 0 && ((uintptr_t)labels % 16) == 0;
  const size_t need = ulysses_sp_loss_workspace_bytes(sp, B, Ns);
  if (!workspace || workspace_bytes < need) return ULY_EWORKSPACE;
  const int nblk = blocks_per_rank(n);
  double* psum = static_cast<double*>(workspace);
  long long* pcnt = reinterpret_cast<long long*>(psum + (size_t)sp * nblk);
  hipStream_t st = (hipStream_t)stream;
  if (vec)
    hipLaunchKernelGGL(loss_partial_kernel<true>, dim3((unsigned)nblk, (unsigned)sp), dim3(kLossThreads), 0, st,
                       token_loss, labels, psum, pcnt, n, (long long)ignore_index);
  else
    hipLaunchKernelGGL(loss_partial_kernel<false>, dim3((unsigned)nblk, (unsigned)sp), dim3(kLossThreads), 0, st,
                       token_loss, labels, psum, pcnt, n, (long long)ignore_index);
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(kLossThreads), 0, st, psum, pcnt, nblk, sp, rank_loss,
                     good_tokens, loss);
  return uly_host::launch_status();
}
