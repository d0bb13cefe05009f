// Sequence-sharded <-> head-sharded layout change of sp virtual ranks on one
// device: the data movement of Ulysses' two all-to-alls (HF Transformers docs,
// "Ulysses sequence parallelism", layout diagram).
//
// Both layouts are made of "runs": the Hl*d elements of one (rank, batch row,
// token) in the head-sharded layout are the same Hl*d contiguous elements of
// one (shard, batch row, token, head block) in the sequence-sharded layout.
// A run is R 16-byte chunks (256 B to 1 KiB at the shapes of interest).
//
// The grid carries the coordinates, so a chunk's two addresses cost a few
// integer operations, and consecutive threads write consecutive chunks of
// the output (contiguous writes matter more than contiguous reads here):
//   * seq -> head: blockIdx.z = shard s, blockIdx.y = (rank r, batch row b),
//     x = (token t within the shard, chunk w within the run);
//   * head -> seq: blockIdx.z = shard s, blockIdx.y = batch row b,
//     x = (token t, rank r, chunk w);
// with shifts where R and sp are powers of two, divisions otherwise. The
// reads are contiguous within each run. Every thread moves kUnroll chunks,
// all loads before the first store; loads and stores are non-temporal (the
// data streams through once). A pure copy of bits, exact for any content.
// One launch can move up to kMaxBatch tensors of the same shape (q, k and v
// of one exchange): blockIdx.z then also carries the tensor, which saves the
// launch's ramp and drain per extra tensor (a few microseconds, a quarter of
// a 64 MiB tensor's time).

#include "common.h"

namespace {

constexpr int kThreads = 256;
// 2 chunks per thread (8 KB per workgroup): against 4, the 64 MiB tensors of
// the llama7b workload move 8-16% faster and the 1 GiB ones 3% (cold inputs,
// same box; 8 per thread, or 512 and 1024 threads, ran slower)
constexpr int kUnroll = 2;
constexpr uint32_t kChunksPerBlock = kThreads * kUnroll;
constexpr int kMaxBatch = 4;

// the tensors of one launch; blockIdx.z = tensor * sp + shard
struct PermutePtrs {
  const uint4* src[kMaxBatch];
  uint4* dst[kMaxBatch];
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// 16-byte non-temporal load and store
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void st_nt(uint4* p, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

struct PermuteGeom {
  uint32_t R;        // 16-byte chunks per run
  int32_t rshift;    // log2(R) when R is a power of two, else -1
  int32_t spshift;   // log2(sp) when sp is a power of two, else -1
  uint32_t Ns;       // tokens per shard (N / sp)
  uint32_t B;
  uint32_t sp;
  uint32_t rb_count; // sp * B
  uint64_t run16;    // R (as 64-bit)
};

// seq -> head: blockIdx.y = (rank r, batch row b), x over (t, w) of the
// head-sharded output, which is contiguous in that order.
__global__ __launch_bounds__(kThreads) void permute_seq_to_head(PermutePtrs ptrs, PermuteGeom g) {
  const uint32_t tensor = blockIdx.z / g.sp, s = blockIdx.z - tensor * g.sp;
  const uint4* __restrict__ src = ptrs.src[tensor];
  uint4* __restrict__ dst = ptrs.dst[tensor];
  const uint32_t slab = g.Ns * g.R;
  for (uint32_t rb = blockIdx.y; rb < g.rb_count; rb += gridDim.y) {
    const uint32_t r = rb / g.B, b = rb - (rb / g.B) * g.B;
    // output run (r*B + b)*N + s*Ns + t; input run ((s*B + b)*Ns + t)*sp + r
    const uint64_t out0 = ((uint64_t)rb * g.sp + s) * g.Ns * g.run16;
    const uint64_t in0 = (((uint64_t)s * g.B + b) * g.Ns * g.sp + r) * g.run16;
    const uint64_t in_tstride = (uint64_t)g.sp * g.run16;
    uint4 buf[kUnroll];
    const uint32_t c0 = blockIdx.x * kChunksPerBlock + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t c = c0 + j * kThreads;
      if (c < slab) {
        const uint32_t t = g.rshift >= 0 ? c >> g.rshift : c / g.R;
        const uint32_t w = c - t * g.R;
        buf[j] = ld_nt(src + in0 + (uint64_t)t * in_tstride + w);
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t c = c0 + j * kThreads;
      if (c < slab) st_nt(dst + out0 + c, buf[j]);
    }
  }
}

// head -> seq: blockIdx.y = batch row b, x over (t, r, w) of the
// sequence-sharded output, which is contiguous in that order.
__global__ __launch_bounds__(kThreads) void permute_head_to_seq(PermutePtrs ptrs, PermuteGeom g) {
  const uint32_t tensor = blockIdx.z / g.sp, s = blockIdx.z - tensor * g.sp;
  const uint4* __restrict__ src = ptrs.src[tensor];
  uint4* __restrict__ dst = ptrs.dst[tensor];
  const uint32_t slab = g.Ns * g.sp * g.R;
  for (uint32_t b = blockIdx.y; b < g.B; b += gridDim.y) {
    // output run ((s*B + b)*Ns + t)*sp + r; input run (r*B + b)*N + s*Ns + t
    const uint64_t out0 = ((uint64_t)s * g.B + b) * g.Ns * g.sp * g.run16;
    const uint64_t in0 = ((uint64_t)b * g.sp * g.Ns + (uint64_t)s * g.Ns) * g.run16;
    const uint64_t in_rstride = (uint64_t)g.B * g.sp * g.Ns * g.run16;  // one rank further
    uint4 buf[kUnroll];
    const uint32_t c0 = blockIdx.x * kChunksPerBlock + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t c = c0 + j * kThreads;
      if (c < slab) {
        const uint32_t tr = g.rshift >= 0 ? c >> g.rshift : c / g.R;
        const uint32_t w = c - tr * g.R;
        const uint32_t t = g.spshift >= 0 ? tr >> g.spshift : tr / g.sp;
        const uint32_t r = tr - t * g.sp;
        buf[j] = ld_nt(src + in0 + (uint64_t)r * in_rstride + (uint64_t)t * g.run16 + w);
      }
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const uint32_t c = c0 + j * kThreads;
      if (c < slab) st_nt(dst + out0 + c, buf[j]);
    }
  }
}

// byte ranges [a, a + n) and [b, b + n) overlap
inline bool overlaps(const void* a, const void* b, uint64_t n) {
  const uint8_t* a8 = static_cast<const uint8_t*>(a);
  const uint8_t* b8 = static_cast<const uint8_t*>(b);
  return a8 < b8 + n && b8 < a8 + n;
}

template <bool kSeqToHead>
int launch_permute(const void* const* src, void* const* dst, int n, int B, int N, int H, int d, int sp,
                   int dtype, void* stream) {
  if (!src || !dst || n < 1 || n > kMaxBatch) return ULY_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!src[i] || !dst[i]) return ULY_EINVAL;
  if (B <= 0 || N <= 0 || H <= 0 || d <= 0 || sp <= 0) return ULY_EINVAL;
  if (!uly_host::dtype_ok(dtype) || !uly_host::head_dim_ok(d)) return ULY_EUNSUPPORTED;
  if (N % sp || H % sp) return ULY_ESHAPE;
  const uint64_t esz = uly_host::elem_size(dtype);
  const uint64_t Hl = (uint64_t)(H / sp);
  const uint64_t total_bytes = (uint64_t)B * N * H * d * esz;
  // an output may overlap no input and no other output; 16-byte accesses need
  // 16-byte aligned buffers (runs are multiples of 16 bytes)
  for (int i = 0; i < n; ++i) {
    if (((uintptr_t)src[i] | (uintptr_t)dst[i]) & 15) return ULY_EINVAL;
    for (int j = 0; j < n; ++j) {
      if (overlaps(dst[i], src[j], total_bytes)) return ULY_EINVAL;
      if (j != i && overlaps(dst[i], dst[j], total_bytes)) return ULY_EINVAL;
    }
  }

  PermuteGeom g;
  const uint64_t run_bytes = Hl * d * esz;
  g.R = (uint32_t)(run_bytes / 16);
  g.rshift = g.spshift = -1;
  for (int k = 0; k < 32; ++k) {
    if ((1u << k) == g.R) g.rshift = k;
    if ((1u << k) == (uint32_t)sp) g.spshift = k;
  }
  g.Ns = (uint32_t)(N / sp);
  g.B = (uint32_t)B;
  g.sp = (uint32_t)sp;
  g.run16 = g.R;
  // a slab of output chunks is indexed in 32 bits; sp is the grid's z
  const uint64_t slab = kSeqToHead ? (uint64_t)g.Ns * g.R : (uint64_t)g.Ns * g.sp * g.R;
  if (slab + kChunksPerBlock >= (1ULL << 32) || sp > 65535 || (uint64_t)sp * B >= (1ULL << 32)) return ULY_ESHAPE;
  if ((uint64_t)n * sp > 65535) return ULY_ESHAPE;  // the grid's z
  g.rb_count = (uint32_t)(sp * B);
  const uint64_t bx = (slab + kChunksPerBlock - 1) / kChunksPerBlock;
  if (bx > 0x7fffffffULL) return ULY_ESHAPE;
  const uint32_t ny = kSeqToHead ? g.rb_count : g.B;
  const dim3 grid((unsigned)bx, ny < 65535u ? ny : 65535u, (unsigned)(n * sp));
  PermutePtrs ptrs{};
  for (int i = 0; i < n; ++i) {
    ptrs.src[i] = static_cast<const uint4*>(src[i]);
    ptrs.dst[i] = static_cast<uint4*>(dst[i]);
  }
  if (kSeqToHead)
    hipLaunchKernelGGL(permute_seq_to_head, grid, dim3(kThreads), 0, (hipStream_t)stream, ptrs, g);
  else
    hipLaunchKernelGGL(permute_head_to_seq, grid, dim3(kThreads), 0, (hipStream_t)stream, ptrs, g);
  return uly_host::launch_status();
}

}  // namespace

extern "C" int ulysses_seq_to_head(const void* x_seq, void* x_head, int B, int N, int H, int d,
                                   int sp, int dtype, void* stream) {
  return launch_permute<true>(&x_seq, &x_head, 1, B, N, H, d, sp, dtype, stream);
}

extern "C" int ulysses_head_to_seq(const void* x_head, void* x_seq, int B, int N, int H, int d,
                                   int sp, int dtype, void* stream) {
  return launch_permute<false>(&x_head, &x_seq, 1, B, N, H, d, sp, dtype, stream);
}

extern "C" int ulysses_seq_to_head_n(const void* const* x_seq, void* const* x_head, int n, int B, int N,
                                     int H, int d, int sp, int dtype, void* stream) {
  return launch_permute<true>(x_seq, x_head, n, B, N, H, d, sp, dtype, stream);
}

extern "C" int ulysses_head_to_seq_n(const void* const* x_head, void* const* x_seq, int n, int B, int N,
                                     int H, int d, int sp, int dtype, void* stream) {
  return launch_permute<false>(x_head, x_seq, n, B, N, H, d, sp, dtype, stream);
}

extern "C" const char* ulysses_status_string(int status) {
  switch (status) {
    case ULY_OK: return "ok";
    case ULY_EINVAL: return "invalid argument (null pointer, size <= 0, overlapping or misaligned buffers, or step out of range)";
    case ULY_ESHAPE: return "a size condition of the call fails (N % sp, H % sp, max_doc_len > N, or a size limit listed in ulysses.h)";
    case ULY_EUNSUPPORTED: return "unsupported dtype or head dimension (d must be 64 or 128)";
    case ULY_EWORKSPACE: return "workspace missing or too small";
    case ULY_EHIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}
