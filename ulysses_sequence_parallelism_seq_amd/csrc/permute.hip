// Sequence-sharded <-> head-sharded layout change of sp virtual ranks on one
// device: the data movement of Ulysses' two all-to-alls (HF Transformers docs,
// "Ulysses sequence parallelism", layout diagram).
//
// Both layouts are made of "runs": the Hl*d elements of one (rank, batch row,
// token) in the head-sharded layout are the same Hl*d contiguous elements of
// one (shard, batch row, token, head block) in the sequence-sharded layout.
// A run is 256 B to 1 KiB at the shapes of interest, so both the reads and
// the writes are whole contiguous segments. Every thread moves U 16-byte
// chunks: all U loads are issued before the first store (memory-level
// parallelism), and consecutive threads touch consecutive chunks (coalescing).
// The kernel is a pure copy of bits and therefore exact for any content.

#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct PermuteGeom {
  uint32_t R;   // 16-byte chunks per run
  uint32_t N;   // full sequence length
  uint32_t Ns;  // N / sp
  uint32_t B;
  uint32_t sp;
  uint64_t run_bytes;
  uint64_t total_chunks;
};

// Byte offset of the source run feeding output run q.
template <bool kSeqToHead>
__device__ __forceinline__ uint64_t source_run(uint32_t q, const PermuteGeom& g) {
  if (kSeqToHead) {
    // output x_head[r][b][n], n = s*Ns + t  <-  input x_seq[s][b][t][r-th head block]
    uint32_t n = q % g.N;
    uint32_t rb = q / g.N;
    uint32_t b = rb % g.B;
    uint32_t r = rb / g.B;
    uint32_t s = n / g.Ns;
    uint32_t t = n - s * g.Ns;
    uint64_t token = ((uint64_t)s * g.B + b) * g.Ns + t;  // row of x_seq
    return (token * g.sp + r) * g.run_bytes;
  } else {
    // output x_seq[s][b][t][r-th head block]  <-  input x_head[r][b][s*Ns + t]
    uint32_t r = q % g.sp;
    uint32_t rest = q / g.sp;
    uint32_t t = rest % g.Ns;
    rest /= g.Ns;
    uint32_t b = rest % g.B;
    uint32_t s = rest / g.B;
    uint64_t token = ((uint64_t)r * g.B + b) * g.N + (uint64_t)s * g.Ns + t;  // row of x_head
    return token * g.run_bytes;
  }
}

template <bool kSeqToHead>
__global__ __launch_bounds__(kThreads) void permute_runs(const uint8_t* __restrict__ src,
                                                         uint8_t* __restrict__ dst, PermuteGeom g) {
  const uint64_t base = (uint64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  uint4 buf[kUnroll];
  uint64_t dst_off[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const uint64_t c = base + (uint64_t)j * kThreads;
    dst_off[j] = c * 16;
    if (c < g.total_chunks) {
      const uint32_t q = (uint32_t)(c / g.R);
      const uint32_t w = (uint32_t)(c - (uint64_t)q * g.R);
      buf[j] = *reinterpret_cast<const uint4*>(src + source_run<kSeqToHead>(q, g) + (uint64_t)w * 16);
    }
  }
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const uint64_t c = base + (uint64_t)j * kThreads;
    if (c < g.total_chunks) *reinterpret_cast<uint4*>(dst + dst_off[j]) = buf[j];
  }
}

template <bool kSeqToHead>
int launch_permute(const void* src, void* dst, int B, int N, int H, int d, int sp, int dtype,
                   void* stream) {
  if (!src || !dst) return ULY_EINVAL;
  if (B <= 0 || N <= 0 || H <= 0 || d <= 0 || sp <= 0) return ULY_EINVAL;
  if (!uly_host::dtype_ok(dtype) || !uly_host::head_dim_ok(d)) return ULY_EUNSUPPORTED;
  if (N % sp || H % sp) return ULY_ESHAPE;
  const uint64_t esz = uly_host::elem_size(dtype);
  const uint64_t Hl = (uint64_t)(H / sp);
  const uint64_t total_bytes = (uint64_t)B * N * H * d * esz;
  // Run indices are 32-bit: sp * B * N runs.
  if ((uint64_t)sp * B * N >= (1ULL << 32)) return ULY_ESHAPE;
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  uint8_t* d8 = static_cast<uint8_t*>(dst);
  if (s8 < d8 + total_bytes && d8 < s8 + total_bytes) return ULY_EINVAL;  // overlap

  PermuteGeom g;
  g.run_bytes = Hl * d * esz;
  g.R = (uint32_t)(g.run_bytes / 16);
  g.N = (uint32_t)N;
  g.Ns = (uint32_t)(N / sp);
  g.B = (uint32_t)B;
  g.sp = (uint32_t)sp;
  g.total_chunks = total_bytes / 16;
  const uint64_t per_block = (uint64_t)kThreads * kUnroll;
  const uint64_t blocks = (g.total_chunks + per_block - 1) / per_block;
  if (blocks > 0x7fffffffULL) return ULY_ESHAPE;
  hipLaunchKernelGGL(permute_runs<kSeqToHead>, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, s8, d8, g);
  return uly_host::launch_status();
}

}  // namespace

extern "C" int ulysses_seq_to_head(const void* x_seq, void* x_head, int B, int N, int H, int d,
                                   int sp, int dtype, void* stream) {
  return launch_permute<true>(x_seq, x_head, B, N, H, d, sp, dtype, stream);
}

extern "C" int ulysses_head_to_seq(const void* x_head, void* x_seq, int B, int N, int H, int d,
                                   int sp, int dtype, void* stream) {
  return launch_permute<false>(x_head, x_seq, B, N, H, d, sp, dtype, stream);
}

extern "C" const char* ulysses_status_string(int status) {
  switch (status) {
    case ULY_OK: return "ok";
    case ULY_EINVAL: return "invalid argument (null pointer, size <= 0, or overlapping buffers)";
    case ULY_ESHAPE: return "inconsistent shape (N % sp, H % sp, max_doc_len > N, or size limits)";
    case ULY_EUNSUPPORTED: return "unsupported dtype or head dimension (d must be 64 or 128)";
    case ULY_EWORKSPACE: return "workspace missing or too small";
    case ULY_EHIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}
