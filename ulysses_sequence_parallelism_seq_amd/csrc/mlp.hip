// Tiled MLP of ALST (TiledMLP) on gfx950 matrix cores (bf16 operands, fp32
// accumulation), and the ulysses_tiled_mlp_* entry points.
//
// What it computes (HF guide "Ulysses sequence parallelism" (deepspeed_alst),
// the paragraph after the layout diagram: ALST pairs Ulysses with TiledMLP;
// the jianying88 page's account of the layout: after the second all-to-all
// the FFN runs locally on each rank's own token shard). Taken as the SwiGLU
// FFN of the Llama-style model the workloads are shaped like,
//   G = X Wg^T,  U = X Wu^T,  A = silu(G) * U,  Y = A Wd^T,
// computed over the rank's tokens in tiles of `tile` tokens so that only one
// tile's [tile, I] intermediates exist at a time. The backward recomputes
// them tile by tile and accumulates the weight gradients over the tiles:
//   dA = dY Wd,  dWd += dY^T A,  dG = dA * U * silu'(G),  dU = dA * silu(G),
//   dX = dG Wg + dU Wu,  dWg += dG^T X,  dWu += dU^T X.
//
// Every product is one GEMM kernel with a fused epilogue:
//   * 256 x 256 output tile per workgroup of 8 waves (2 along M x 4 along N,
//     each wave 128 x 64 = 4 x 2 blocks of the 32x32x16 bf16 MFMA), one
//     workgroup per CU (two waves per SIMD);
//   * K in tiles of 64, double-buffered in LDS by direct-to-LDS loads (tile
//     t+1 in flight during the MFMAs of tile t, one barrier per tile); the two
//     stages are separate arrays addressed by name;
//   * an operand whose K index is contiguous in memory ([rows][k], e.g. X,
//     or W when the product takes W^T) is staged as [rows][64 k] and read with
//     16-byte LDS reads; an operand whose K index is the strided one
//     ([k][rows], e.g. W in dY Wd, or dY and X in the weight gradients) is
//     staged as it lies in memory, [64 k][rows], and read with the
//     transposing LDS read addressed so that its k order is the 16-byte
//     read's (the two operands of an MFMA must agree on it): no transposed
//     copy of any tensor is made;
//   * loads go through buffer resources that end at the operand's last row,
//     so rows past a ragged token count read as zero;
//   * workgroups are dealt to the 8 XCDs round-robin; the tile order gives
//     each XCD a contiguous run of tiles, M fastest in groups of 8 row tiles,
//     so the workgroups on one XCD share A and B panels in its L2.

#include <math.h>

#include <initializer_list>

#include "common.h"

namespace {

using namespace uly;

constexpr int kBM = 256, kBN = 256, kBKt = 64;  // workgroup tile, K tile
constexpr int kThreads = 512;                    // 8 waves
constexpr int kGroupM = 8;                       // row tiles per tile group

enum Epilogue : int {
  kEpiStoreBf16 = 0,  // C -> bf16
  kEpiGateUp = 1,     // forward: A = silu(G) * U -> bf16
  kEpiGateUpSave = 2, // backward recompute: A, U * silu'(G) and silu(G) -> bf16
  kEpiDGrad = 3,      // backward: dG = dA * (U * silu'(G)), dU = dA * silu(G), in place of the two factors
  kEpiAccF32 = 4,     // weight gradients: C (+)= acc in fp32
};

struct GemmArgs {
  // Up to two (A, B) pairs whose products are summed (dX = dG Wg + dU Wu).
  // For the gate/up products b[0] is Wg and b[1] is Wu, both against a[0].
  const bf16* a[2];
  const bf16* b[2];
  int ksize[2];
  int npairs;
  int lda, ldb;  // elements between consecutive rows of the stored operand
  int M, N;
  int tiles_m, tiles_n;
  void* c;  // bf16 or float output
  int ldc;
  bf16* act;  // A (gate/up epilogues)
  bf16* g;    // U * silu'(G), then dG
  bf16* u;    // silu(G), then dU
  int accumulate;
};

// silu(z) = z sigmoid(z), sigmoid(z) = 1 / (1 + 2^(-z log2 e)) on the
// hardware exp2 and reciprocal; z -> -inf gives 1 / inf = 0.
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * kLog2e));
}

// Four bf16 values, rounded to nearest even, as one 8-byte store; and back.
__device__ __forceinline__ void st_bf16x4(bf16* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void ld_bf16x4(const bf16* p, float* v) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
}

// Tile order: blockIdx -> XCD x = blockIdx % 8 (round-robin dispatch); XCD x
// takes the contiguous run [start_x, start_x + count_x) of the tiles (a
// bijection for any tile count), numbered M fastest within groups of
// kGroupM row tiles.
__device__ __forceinline__ void tile_of(const GemmArgs& p, int& bm, int& bn) {
  const int total = p.tiles_m * p.tiles_n;
  const int i = blockIdx.x;
  const int x = i & 7, per = total >> 3, rem = total & 7;
  const int L = x * per + min(x, rem) + (i >> 3);
  const int per_group = kGroupM * p.tiles_n;
  const int grp = L / per_group;
  const int first = grp * kGroupM;
  const int gm = min(kGroupM, p.tiles_m - first);
  const int r = L - grp * per_group;
  bm = first + r % gm;
  bn = r / gm;
}

// kAK: A stored [M][lda] (K contiguous), else [K][lda] (M contiguous).
// kBK: B stored [N][ldb] (K contiguous), else [K][ldb] (N contiguous).
template <bool kAK, bool kBK, int kEpi>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr bool kGateUp = kEpi == kEpiGateUp || kEpi == kEpiGateUpSave;
  // accumulator blocks transposed (the B fragment as the MFMA's first
  // operand): a lane then holds four consecutive output columns per group of
  // four elements, and the epilogue moves 8 or 16 bytes per access. The
  // recompute epilogue, which writes three bf16 arrays, keeps the plain
  // blocks (a lane = one column): there the 32 rows x 16 bytes that each
  // transposed store touches cost more than its fewer instructions save.
  constexpr bool kTransAcc = kEpi != kEpiGateUpSave;
  constexpr int TILE = kBM * kBKt;  // bf16 elements of one staged operand tile (both layouts)
  __shared__ __attribute__((aligned(16))) bf16 a0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 b0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 a1s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 b1s[TILE];

  int bm, bn;
  tile_of(p, bm, bn);
  const int m0 = bm * kBM;
  const int n0 = bn * (kGateUp ? kBN / 2 : kBN);  // gate/up: 128 output units, 128 rows of Wg and of Wu

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wm = w >> 2, wn = w & 3;
  FragOffsets<64> fo64;     // 16-byte reads of K-contiguous tiles
  NatTrOffsets<128> nt128;  // transposing reads of K-strided tiles, same k order
  fo64.init(lane);
  nt128.init(lane);

  const uint32_t arow = (uint32_t)p.lda * 2u, brow = (uint32_t)p.ldb * 2u;
  // Direct-to-LDS staging. A K-contiguous operand tile is 256 rows of 64 k
  // (RowTile<64>); a K-strided one is 64 rows of k, stored as two [64][128]
  // halves (RowTile<128>). The gate/up B tile is 128 rows of Wg then 128 of Wu.
  // Only the loaders the layout needs are used; the others are dead code.
  TileDma<64, kBM, 8> dma_a_rows, dma_b_rows;
  TileDma<128, kBKt, 8> dma_a_k, dma_b_k;
  TileDma<64, kBN / 2, 8> dma_b_half;
  dma_a_rows.init(w, lane, arow);
  dma_a_k.init(w, lane, arow);
  dma_b_rows.init(w, lane, brow);
  dma_b_k.init(w, lane, brow);
  dma_b_half.init(w, lane, brow);

  int ntk[2];
  ntk[0] = (p.ksize[0] + kBKt - 1) / kBKt;
  ntk[1] = p.npairs > 1 ? (p.ksize[1] + kBKt - 1) / kBKt : 0;
  const int ntiles = ntk[0] + ntk[1];

  auto load = [&](int t, bf16* as, bf16* bs) {
    const int pi = t < ntk[0] ? 0 : 1;
    const int k0 = (t - (pi ? ntk[0] : 0)) * kBKt;
    const int K = p.ksize[pi];
    const bf16* A = p.a[pi];
    const bf16* B = p.b[pi];
    if constexpr (kAK) {
      const int rows = min(p.M - m0, kBM);
      dma_a_rows.issue(make_rsrc(A + (size_t)m0 * p.lda + k0, (long long)rows * arow), as);
    } else {
      const int rows = min(K - k0, kBKt);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        dma_a_k.issue(make_rsrc(A + (size_t)k0 * p.lda + m0 + 128 * s, (long long)rows * arow), as + s * kBKt * 128);
    }
    if constexpr (kGateUp) {
      dma_b_half.issue(make_rsrc(p.b[0] + (size_t)n0 * p.ldb + k0, (long long)(kBN / 2) * brow), bs);
      dma_b_half.issue(make_rsrc(p.b[1] + (size_t)n0 * p.ldb + k0, (long long)(kBN / 2) * brow), bs + (kBN / 2) * kBKt);
    } else if constexpr (kBK) {
      dma_b_rows.issue(make_rsrc(B + (size_t)n0 * p.ldb + k0, (long long)kBN * brow), bs);
    } else {
      const int rows = min(K - k0, kBKt);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        dma_b_k.issue(make_rsrc(B + (size_t)k0 * p.ldb + n0 + 128 * s, (long long)rows * brow), bs + s * kBKt * 128);
    }
  };

  // operand fragments of one k-step: A blocks mb = 0..3 (rows 128 wm + 32 mb),
  // B blocks nb = 0..1 (rows 64 wn + 32 nb; gate/up: 32 wn of Wg and of Wu)
  auto frag_a = [&](const bf16* as, int mb, int kk) -> bf16x8 {
    if constexpr (kAK) {
      return as_bf16x8(lds_ld16(as, fo64.row_frag(4 * wm + mb, kk)));
    } else {
      return a_from_rows_nat<128>(as + wm * kBKt * 128, nt128, kk, mb);
    }
  };
  auto frag_b = [&](const bf16* bs, int nb, int kk) -> bf16x8 {
    const int nrow = kGateUp ? nb * (kBN / 2) + 32 * wn : 64 * wn + 32 * nb;
    if constexpr (kGateUp || kBK) {
      return as_bf16x8(lds_ld16(bs, fo64.row_frag(nrow / 32, kk)));
    } else {
      return a_from_rows_nat<128>(bs + (nrow / 128) * kBKt * 128, nt128, kk, (nrow % 128) / 32);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;

  auto compute = [&](const bf16* as, const bf16* bs) {
    bf16x8 fa[2][4], fb[2][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fa[0][mb] = frag_a(as, mb, 0);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) fb[0][nb] = frag_b(bs, nb, 0);
#pragma unroll
    for (int kk = 0; kk < kBKt / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < kBKt / 16) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) fa[cur ^ 1][mb] = frag_a(as, mb, kk + 1);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) fb[cur ^ 1][nb] = frag_b(bs, nb, kk + 1);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = kTransAcc ? mfma32(fb[cur][nb], fa[cur][mb], acc[mb][nb])
                                  : mfma32(fa[cur][mb], fb[cur][nb], acc[mb][nb]);
    }
  };

  // one K tile: the next tile's loads go out first, then this tile's MFMAs;
  // the barrier after the wait makes the next stage visible and frees this one
  auto step = [&](int t, const bf16* as, const bf16* bs, bf16* an, bf16* bn_) {
    if (t + 1 < ntiles) load(t + 1, an, bn_);
    compute(as, bs);
    wait_vmem();
    __syncthreads();
  };
  load(0, a0s, b0s);
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(t, a0s, b0s, a1s, b1s);
    if (t + 1 < ntiles) step(t + 1, a1s, b1s, a0s, b0s);
  }

  if constexpr (!kTransAcc) {
    // ---- recompute epilogue, plain blocks: element i of acc[mb][nb] in lane l
    // is row m0 + 128 wm + 32 mb + 8 (i / 4) + 4 half + i % 4 and column
    // (intermediate unit) n0 + 32 wn + l % 32, of Wg's rows (nb = 0) and Wu's (nb = 1).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 128 * wm + 32 * mb + 8 * (i >> 2) + 4 * half + (i & 3);
        if (m >= p.M) continue;
        const size_t o = (size_t)m * p.ldc + n0 + 32 * wn + l32;
        const float gv = acc[mb][0][i], uv = acc[mb][1][i];
        const float s = sigmoidf_(gv);
        const float silu = gv * s;
        p.act[o] = (bf16)(silu * uv);
        // the backward's two factors, formed from the fp32 G: silu' has a
        // zero (near G = -1.28) where G's bf16 rounding would become a large
        // relative error of dG; rounding the factor itself costs 2^-8 of it
        p.g[o] = (bf16)(uv * s * (1.0f + gv * (1.0f - s)));
        p.u[o] = (bf16)silu;
      }
    }
    return;
  }
  // ---- epilogue. The MFMAs take the B fragment as their first operand, so
  // acc[mb][nb] holds the block transposed: element i of lane l is row
  // m0 + 128 wm + 32 mb + l % 32 and column 8 (i / 4) + 4 half + i % 4 of
  // block nb. Each group of four elements is four consecutive columns of one
  // row, read and written 8 bytes (bf16) or 16 bytes (fp32) at a time.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + 128 * wm + 32 * mb + l32;
    if (m >= p.M) continue;
    const size_t row = (size_t)m * p.ldc;
    if constexpr (kGateUp) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float a4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = acc[mb][0][4 * gq + j], uv = acc[mb][1][4 * gq + j];
          a4[j] = gv * sigmoidf_(gv) * uv;
        }
        st_bf16x4(p.act + row + n0 + 32 * wn + 8 * gq + 4 * half, a4);  // intermediate units
      }
    } else {
      // column of group gq of block nb; the epilogues that read memory issue
      // all of the block row's loads before its first store (a store may
      // alias a later load, so the compiler would otherwise wait for each
      // load in turn)
      auto col = [&](int gq, int nb) { return row + n0 + 64 * wn + 32 * nb + 8 * gq + 4 * half; };
      if constexpr (kEpi == kEpiStoreBf16) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const float v4[4] = {acc[mb][nb][4 * gq], acc[mb][nb][4 * gq + 1], acc[mb][nb][4 * gq + 2],
                                 acc[mb][nb][4 * gq + 3]};
            st_bf16x4(static_cast<bf16*>(p.c) + col(gq, nb), v4);
          }
      } else if constexpr (kEpi == kEpiDGrad) {
        float g4[4][2][4], u4[4][2][4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            ld_bf16x4(p.g + col(gq, nb), g4[gq][nb]);
            ld_bf16x4(p.u + col(gq, nb), u4[gq][nb]);
          }
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v = acc[mb][nb][4 * gq + j];
              g4[gq][nb][j] *= v;  // dG = dA * U * silu'(G)
              u4[gq][nb][j] *= v;  // dU = dA * silu(G)
            }
            st_bf16x4(p.g + col(gq, nb), g4[gq][nb]);
            st_bf16x4(p.u + col(gq, nb), u4[gq][nb]);
          }
      } else {  // kEpiAccF32
        float* c = static_cast<float*>(p.c);
        float4 old[4][2];
        if (p.accumulate) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) old[gq][nb] = *reinterpret_cast<const float4*>(c + col(gq, nb));
        }
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            float4 r = make_float4(acc[mb][nb][4 * gq], acc[mb][nb][4 * gq + 1], acc[mb][nb][4 * gq + 2],
                                   acc[mb][nb][4 * gq + 3]);
            if (p.accumulate) {
              const float4 o = old[gq][nb];
              r = make_float4(o.x + r.x, o.y + r.y, o.z + r.z, o.w + r.w);
            }
            *reinterpret_cast<float4*>(c + col(gq, nb)) = r;
          }
      }
    }
  }
}

// ---------------------------------------------------------------- launching

template <bool kAK, bool kBK, int kEpi>
int launch_gemm(GemmArgs p, hipStream_t st) {
  constexpr bool kGateUp = kEpi == kEpiGateUp || kEpi == kEpiGateUpSave;
  p.tiles_m = (p.M + kBM - 1) / kBM;
  p.tiles_n = p.N / (kGateUp ? kBN / 2 : kBN);
  const long long blocks = (long long)p.tiles_m * p.tiles_n;
  if (blocks <= 0) return ULY_OK;
  if (blocks > 0x7fffffffLL) return ULY_ESHAPE;
  hipLaunchKernelGGL((gemm_bf16_kernel<kAK, kBK, kEpi>), dim3((unsigned)blocks), dim3(kThreads), 0, st, p);
  return uly_host::launch_status();
}

GemmArgs gemm_args(int M, int N, const bf16* a, int lda, const bf16* b, int ldb, int K) {
  GemmArgs p{};
  p.a[0] = a;
  p.b[0] = b;
  p.a[1] = p.b[1] = nullptr;
  p.ksize[0] = K;
  p.ksize[1] = 0;
  p.npairs = 1;
  p.lda = lda;
  p.ldb = ldb;
  p.M = M;
  p.N = N;
  return p;
}

struct MlpGeom {
  int T, h, I, tile;
};

// Host-side checks shared by the entry points (all before any launch); the workspace holds three
// [tile][I] bf16 arrays of one tile: A, then U * silu'(G) and silu(G) (the
// backward's factors, overwritten by dG and dU).
int check_mlp(int tokens, int hidden, int inter, int tile) {
  if (tokens <= 0 || hidden <= 0 || inter <= 0 || tile <= 0) return ULY_EINVAL;
  if (hidden % kBN || inter % kBN) return ULY_ESHAPE;
  // 32-bit buffer ranges and lane offsets: a staged tile spans < 2 GiB
  const long long wide = hidden > inter ? hidden : inter;
  if ((long long)kBM * 2 * wide >= (1LL << 31)) return ULY_ESHAPE;
  // every launch's grid (row tiles x column tiles) fits, so no call stops
  // with an error after some of its launches were enqueued
  const long long rows = tile < tokens ? tile : tokens;
  const long long tall = rows > wide ? rows : wide;
  if ((tall + kBM - 1) / kBM * (wide / (kBN / 2)) > 0x7fffffffLL) return ULY_ESHAPE;
  return ULY_OK;
}

// 16-byte accesses (direct-to-LDS loads, the epilogues' 8- and 16-byte
// stores) need 16-byte aligned buffers
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if ((uintptr_t)q & 15) return false;
  return true;
}

size_t mlp_ws_bytes(int tokens, int inter, int tile) {
  const long long t = tile < tokens ? tile : tokens;
  return 3 * (size_t)t * inter * sizeof(bf16);
}

}  // namespace

extern "C" size_t ulysses_tiled_mlp_workspace_bytes(int tokens, int hidden, int inter, int tile) {
  if (check_mlp(tokens, hidden, inter, tile) != ULY_OK) return 0;
  return mlp_ws_bytes(tokens, inter, tile);
}

extern "C" int ulysses_tiled_mlp_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                                     void* y, void* workspace, size_t workspace_bytes, int tokens, int hidden,
                                     int inter, int tile, void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !y) return ULY_EINVAL;
  if (!aligned16({x, w_gate, w_up, w_down, y, workspace})) return ULY_EINVAL;
  const int rc = check_mlp(tokens, hidden, inter, tile);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < mlp_ws_bytes(tokens, inter, tile)) return ULY_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bf16* X = static_cast<const bf16*>(x);
  bf16* act = static_cast<bf16*>(workspace);
  for (int t0 = 0; t0 < tokens; t0 += tile) {
    const int Tt = tokens - t0 < tile ? tokens - t0 : tile;
    // A = silu(X Wg^T) * (X Wu^T): [Tt][I]
    GemmArgs p = gemm_args(Tt, inter, X + (size_t)t0 * hidden, hidden, static_cast<const bf16*>(w_gate), hidden,
                           hidden);
    p.b[1] = static_cast<const bf16*>(w_up);
    p.act = act;
    p.ldc = inter;
    int r = launch_gemm<true, true, kEpiGateUp>(p, st);
    if (r != ULY_OK) return r;
    // Y = A Wd^T: [Tt][h]
    GemmArgs q = gemm_args(Tt, hidden, act, inter, static_cast<const bf16*>(w_down), inter, inter);
    q.c = static_cast<bf16*>(y) + (size_t)t0 * hidden;
    q.ldc = hidden;
    r = launch_gemm<true, true, kEpiStoreBf16>(q, st);
    if (r != ULY_OK) return r;
  }
  return ULY_OK;
}

extern "C" int ulysses_tiled_mlp_bwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                                     const void* dy, void* dx, float* dw_gate, float* dw_up, float* dw_down,
                                     void* workspace, size_t workspace_bytes, int tokens, int hidden, int inter,
                                     int tile, void* stream) {
  if (!x || !w_gate || !w_up || !w_down || !dy || !dx || !dw_gate || !dw_up || !dw_down) return ULY_EINVAL;
  if (!aligned16({x, w_gate, w_up, w_down, dy, dx, dw_gate, dw_up, dw_down, workspace})) return ULY_EINVAL;
  const int rc = check_mlp(tokens, hidden, inter, tile);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < mlp_ws_bytes(tokens, inter, tile)) return ULY_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bf16* X = static_cast<const bf16*>(x);
  const bf16* Wg = static_cast<const bf16*>(w_gate);
  const bf16* Wu = static_cast<const bf16*>(w_up);
  const bf16* Wd = static_cast<const bf16*>(w_down);
  const bf16* dY = static_cast<const bf16*>(dy);
  const size_t tI = (size_t)(tokens < tile ? tokens : tile) * inter;
  bf16* act = static_cast<bf16*>(workspace);
  bf16* g = act + tI;
  bf16* u = g + tI;
  for (int t0 = 0; t0 < tokens; t0 += tile) {
    const int Tt = tokens - t0 < tile ? tokens - t0 : tile;
    const bf16* Xt = X + (size_t)t0 * hidden;
    const bf16* dYt = dY + (size_t)t0 * hidden;
    // recompute: A and the factors U * silu'(G), silu(G) of the tile
    GemmArgs p = gemm_args(Tt, inter, Xt, hidden, Wg, hidden, hidden);
    p.b[1] = Wu;
    p.act = act;
    p.g = g;
    p.u = u;
    p.ldc = inter;
    int r = launch_gemm<true, true, kEpiGateUpSave>(p, st);
    if (r != ULY_OK) return r;
    // dA = dY Wd (Wd stored [h][I]: K = h strided), then dG, dU in place of the factors
    GemmArgs q = gemm_args(Tt, inter, dYt, hidden, Wd, inter, hidden);
    q.g = g;
    q.u = u;
    q.ldc = inter;
    r = launch_gemm<true, false, kEpiDGrad>(q, st);
    if (r != ULY_OK) return r;
    // dX = dG Wg + dU Wu (Wg, Wu stored [I][h]: K = I strided)
    GemmArgs dxa = gemm_args(Tt, hidden, g, inter, Wg, hidden, inter);
    dxa.a[1] = u;
    dxa.b[1] = Wu;
    dxa.ksize[1] = inter;
    dxa.npairs = 2;
    dxa.c = static_cast<bf16*>(dx) + (size_t)t0 * hidden;
    dxa.ldc = hidden;
    r = launch_gemm<true, false, kEpiStoreBf16>(dxa, st);
    if (r != ULY_OK) return r;
    // dWd (+)= dY^T A: [h][I], K = the tile's tokens (both operands K-strided)
    GemmArgs wd = gemm_args(hidden, inter, dYt, hidden, act, inter, Tt);
    wd.c = dw_down;
    wd.ldc = inter;
    wd.accumulate = t0 > 0;
    r = launch_gemm<false, false, kEpiAccF32>(wd, st);
    if (r != ULY_OK) return r;
    // dWg (+)= dG^T X, dWu (+)= dU^T X: [I][h]
    GemmArgs wg = gemm_args(inter, hidden, g, inter, Xt, hidden, Tt);
    wg.c = dw_gate;
    wg.ldc = hidden;
    wg.accumulate = t0 > 0;
    r = launch_gemm<false, false, kEpiAccF32>(wg, st);
    if (r != ULY_OK) return r;
    GemmArgs wu = wg;
    wu.a[0] = u;
    wu.c = dw_up;
    r = launch_gemm<false, false, kEpiAccF32>(wu, st);
    if (r != ULY_OK) return r;
  }
  return ULY_OK;
}
