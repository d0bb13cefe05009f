// Attention backward on gfx950 matrix cores (bf16 inputs, fp32 accumulation),
// and the ulysses_attn_bwd entry points.
//
// The backward of O = softmax(S) V, S = Q K^T / sqrt(d), recomputes P tile by
// tile from the saved lse (memory-efficient attention keeps only O(N) state;
// congresoia365 article, "El Desafío del Entrenamiento de Secuencias
// Largas"):
//   D_i = sum_c dO_ic O_ic                         (pre-pass, fp32)
//   P = exp(S - lse),  dP = dO V^T,  dS = P * (dP - D)
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO
// with the same mask as the forward (same document; key <= query if causal).
//
// Work split (no atomics, so every output is written by exactly one lane and
// results are bit-reproducible):
//   * dq kernel, query-stationary: a workgroup owns 256 queries (32 per
//     wave, Q and dO resident in registers as MFMA B operands) and walks the
//     64-key K/V tiles of its document (double-buffered in LDS, filled by
//     direct-to-LDS loads). Per tile: S^T = K Q^T and
//     dP^T = V dO^T (lane = query, so lse_i and D_i are per-lane scalars),
//     dS^T in registers, then dQ^T += K^T dS^T (K^T read from the row-major
//     K tile with gfx950's transposing LDS reads).
//   * dkdv kernel, key-stationary: a workgroup of 8 waves owns 128 keys and
//     walks 64-query tiles (Q, dO, lse, D in three LDS stages) from the
//     document end down to its first key (causal). Producer waves compute
//     S = Q K^T, dP = dO V^T (lane = key; K and V resident as B operands),
//     P and dS; consumer waves, one tile behind, accumulate dV^T += dO^T P
//     and dK^T += Q^T dS (64 keys x half the columns each) with the A
//     operands read transposed from the row-major Q and dO tiles; the
//     accumulators hold one key per lane, so the final stores are 4
//     consecutive columns per lane.
// The MFMA k index of a 16-wide step maps to tokens the same way as in the
// forward kernel, so P and dS feed the MFMA straight from the accumulators.

#include <math.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

using namespace uly;

constexpr int kThreads = 256;

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* delta;  // workspace: -D, then lse in log2 units (units * N floats each)
  float* lse2;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  const int* cu;
  int ndoc;
  int nslots;  // tiles per document slot
  int units;   // G * Hl
  int Hl;
  int N;
  int causal;
  float sl2;    // log2(e) / sqrt(d)
  float scale;  // 1 / sqrt(d)
  // ring step only: fp32 running sums of dQ (per query chunk) and dK, dV (per
  // key/value chunk), same layout as dq; the step; ring size and batch rows
  float* dq_acc;
  float* dk_acc;
  float* dv_acc;
  int step, sp, B;
  // persistent launch: the kernel's tile-queue counters (TileQueue), in the
  // workspace; nullptr: one tile per workgroup
  int* sched;
};

template <bool B>
struct RoleTag {
  static constexpr bool value = B;
};

// Ring step geometry of a row g = c * B + b whose chunk c is held by the
// workgroup: chunk c meets chunk c - step (query side, kq) or c + step (key
// side) mod sp. Returns false when the causal mask hides the whole block.
struct RingBlock {
  int other;   // the other chunk's row (its chunk * B + b)
  int causal;  // 1: the causal diagonal block
  bool first, last;
};
__device__ __forceinline__ bool ring_block(const BwdArgs& a, int g, bool query_side, RingBlock& rb) {
  const int c = g / a.B, b = g - (g / a.B) * a.B;
  int oc = query_side ? c - a.step : c + a.step;
  if (oc < 0) oc += a.sp;
  if (oc >= a.sp) oc -= a.sp;
  const int qc = query_side ? c : oc, kc = query_side ? oc : c;  // query chunk, key chunk
  if (a.causal && kc > qc) return false;
  rb.other = oc * a.B + b;
  rb.causal = a.causal && kc == qc;
  rb.first = a.step == 0;
  // a query chunk's last block is key chunk 0 (causal); a key chunk's is query chunk sp - 1
  rb.last = !a.causal ? a.step == a.sp - 1 : (query_side ? a.step == c : a.step == a.sp - 1 - c);
  return true;
}

__device__ __forceinline__ void doc_range(const BwdArgs& a, int doc, int& s, int& e) {
  s = 0;
  e = a.N;
  if (a.cu) {
    s = a.cu[doc];
    e = a.cu[doc + 1];
  }
}

// ------------------------------------------------------------------ D pre-pass
// D[unit][t] = sum_c dO[t][c] * O[t][c], stored negated (the dK/dV kernel
// starts its dP accumulators from it, so its MFMAs leave dP - D); D/8 lanes
// per row, 16 bytes per lane.
// Also lse2[unit][t] = lse[unit][t] * log2(e), the form the dK/dV kernel stages.
// blockIdx.y = unit (g * Hl + h), blockIdx.x = a span of kDeltaPasses * 256 / (D/8)
// tokens; each group of D/8 lanes takes kDeltaPasses rows, all loads (non-temporal:
// O and dO stream through once) issued before the first product.
constexpr int kDeltaPasses = 4;
// Tile-queue counters of a persistent backward, at the end of the workspace:
// the dK/dV kernel's queue (kQueueBytes), then the dQ kernel's.
constexpr int kSchedDq = kQueueBytes / 4;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const bf16* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

template <int D>
__global__ __launch_bounds__(kThreads) void delta_bf16_kernel(const bf16* __restrict__ o,
                                                              const bf16* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              float* __restrict__ delta,
                                                              float* __restrict__ lse2, int N, int Hl,
                                                              long long units, int* __restrict__ sched) {
  // the tile-queue counters of the dK/dV and dQ kernels start at zero
  if (sched && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2 * kQueueInts)
    sched[(threadIdx.x < kQueueInts ? 0 : kSchedDq) + (threadIdx.x % kQueueInts) * kCtrStride] = 0;
  constexpr int LPR = D / 8;              // lanes per row
  constexpr int RPP = kThreads / LPR;     // rows per pass
  const int sub = threadIdx.x % LPR;
  const int t0 = blockIdx.x * (RPP * kDeltaPasses) + threadIdx.x / LPR;
  for (long long unit = blockIdx.y; unit < units; unit += gridDim.y) {
    const long long g = unit / Hl;
    const int h = (int)(unit - g * Hl);
    const size_t tstride = (size_t)Hl * D;  // elements between tokens
    const size_t base = ((size_t)g * N * Hl + h) * D + sub * 8;
    uint4 ov[kDeltaPasses], dv[kDeltaPasses];
#pragma unroll
    for (int p = 0; p < kDeltaPasses; ++p) {
      const int t = t0 + p * RPP;
      if (t < N) {
        ov[p] = ld_nt16(o + base + (size_t)t * tstride);
        dv[p] = ld_nt16(dout + base + (size_t)t * tstride);
      }
    }
#pragma unroll
    for (int p = 0; p < kDeltaPasses; ++p) {
      const int t = t0 + p * RPP;
      float acc = 0.f;
      if (t < N) {
        const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov[p]);
        const uint32_t* dw = reinterpret_cast<const uint32_t*>(&dv[p]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(bf16_bits_to_float(ow[j] & 0xffffu), bf16_bits_to_float(dw[j] & 0xffffu), acc);
          acc = fmaf(bf16_bits_to_float(ow[j] >> 16), bf16_bits_to_float(dw[j] >> 16), acc);
        }
      }
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
      if (t < N && sub == 0) {
        const size_t row = (size_t)unit * N + t;
        delta[row] = -acc;
        lse2[row] = lse[row] * kLog2e;
      }
    }
  }
}

// Ring steps: elements i0 .. i0+3 of an accumulator times s, added to the four
// fp32 running sums at acc (stored as they are at the first step); at the
// last step the sums also go to out as bf16.
__device__ __forceinline__ void add_store4(float* acc, const f32x16& v, int i0, float s, bool first, bf16* out) {
  float4 x = make_float4(v[i0] * s, v[i0 + 1] * s, v[i0 + 2] * s, v[i0 + 3] * s);
  if (!first) {
    const float4 y = *reinterpret_cast<const float4*>(acc);
    x.x += y.x;
    x.y += y.y;
    x.z += y.z;
    x.w += y.w;
  }
  *reinterpret_cast<float4*>(acc) = x;
  if (out) *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
}

// --------------------------------------------------------------------- dq kernel
constexpr int kDqBQ = 256;       // queries per workgroup (32 per wave)
constexpr int kDqThreads = 512;  // 8 waves sharing each K/V tile, one workgroup per CU
constexpr int kDqBK = 64;   // keys per tile

// kRing: one ring step; row g = r * B + b holds rank r's queries, its keys and
// values come from chunk (r - step) mod sp, and dQ is added to dq_acc (written
// to dq at the rank's last step).
template <int D, bool kRing>
__global__ __launch_bounds__(kDqThreads, 1) void attn_dq_bf16_kernel(BwdArgs a) {
  using L = RowTile<D>;
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int TILE = kDqBK * L::RS;  // bf16 elements of one staged tensor
  // K and V of even tiles, then of odd tiles (named stages: see TileDma)
  __shared__ __attribute__((aligned(16))) bf16 k0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 v0s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 k1s[TILE];
  __shared__ __attribute__((aligned(16))) bf16 v1s[TILE];

  __shared__ int s_claim[4];
  TileQueue tq;
  tq.init(a.sched, a.nslots, a.ndoc, a.units);
  TileId tid_;
  while (tq.next(tid_, s_claim)) {
    const int lvl = tid_.lvl, doc = tid_.doc, unit = tid_.unit;
    int s, e;
    doc_range(a, doc, s, e);
    const int q0 = s + (a.nslots - 1 - lvl) * kDqBQ;
    if (q0 >= e) continue;  // the whole workgroup skips the tile

    const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
    const size_t rs = (size_t)a.Hl * D;
    const uint32_t row_bytes = (uint32_t)rs * 2u;
    const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
    size_t kvbase = base;
    int causal = a.causal;
    RingBlock rb{g, a.causal, true, true};
    if constexpr (kRing) {
      if (!ring_block(a, g, true, rb)) continue;  // the whole workgroup skips the tile
      causal = rb.causal;
      kvbase = ((size_t)rb.other * a.N * a.Hl + hd) * D;
    }
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int qi = q0 + 32 * w + l32;
    const bool qvalid = qi < e;
    FragOffsets<D> fo;
    fo.init(lane);

    // Q^T and dO^T as resident B operands (rows past the document end read as zero)
    uint4 qreg[KK], doreg[KK];
    {
      const long long span = (long long)(e - q0) * row_bytes;
      const rsrc_t qr = make_rsrc(a.q + base + (size_t)q0 * rs, span);
      const rsrc_t dr = make_rsrc(a.dout + base + (size_t)q0 * rs, span);
      const uint32_t off = (uint32_t)(32 * w + l32) * row_bytes + (uint32_t)(8 * half) * 2u;
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        qreg[kk] = buf_load16(qr, off + 32u * kk);
        doreg[kk] = buf_load16(dr, off + 32u * kk);
      }
    }
    const float lse2 = qvalid ? a.lse[(size_t)unit * a.N + qi] * kLog2e : 0.f;
    const float ndlt = qvalid ? a.delta[(size_t)unit * a.N + qi] : 0.f;  // -D

    const int kend = causal ? min(e, q0 + kDqBQ) : e;
    const int ntiles = (kend - s + kDqBK - 1) / kDqBK;
    // the last key this wave's queries see (none when they all lie past the
    // document end: their rows are never stored)
    const int wave_klast = q0 + 32 * w >= e ? -1 : causal ? q0 + 32 * w + 31 : e - 1;

    f32x16 dqacc[CB];
  #pragma unroll
    for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
      for (int i = 0; i < 16; ++i) dqacc[cb][i] = 0.f;

    auto rsrc_at = [&](const bf16* p, int kt0) {
      return make_rsrc(p + kvbase + (size_t)kt0 * rs, (long long)(e - kt0) * row_bytes);
    };
    // K/V tiles by direct-to-LDS loads: tile t+1 goes out before the math of
    // tile t and is waited for before its barrier
    TileDma<D, kDqBK, kDqThreads / 64> dma;
    dma.init(w, lane, row_bytes);
    dma.issue(rsrc_at(a.k, s), k0s);
    dma.issue(rsrc_at(a.v, s), v0s);
    wait_vmem();
    __syncthreads();

    auto step = [&](int t, const bf16* ks, const bf16* vs, const bf16* kn, const bf16* vn) {
      const int kt0 = s + t * kDqBK;
      if (t + 1 < ntiles) {
        dma.issue(rsrc_at(a.k, kt0 + kDqBK), kn);
        dma.issue(rsrc_at(a.v, kt0 + kDqBK), vn);
      }

      if (kt0 <= wave_klast) {
        const bool need_mask = (causal && kt0 + kDqBK - 1 > q0) || kt0 + kDqBK > e;
        // one 32-key block at a time: S^T = K Q^T and dP^T = V dO^T (lane = query,
        // element i is key kt0 + blk*32 + 8*(i/4) + 4*half + (i%4)), dS^T, then
        // dQ^T += K^T dS^T with K^T read from the K tile by transposing reads
  #pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          f32x16 sacc, pacc;
  #pragma unroll
          for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
          // K and V fragments read two k-steps ahead of their MFMAs
          auto rd = [&](int kk, uint4* f) {
            const uint32_t off = fo.row_frag(blk, kk);
            f[0] = lds_ld16(ks, off);
            f[1] = lds_ld16(vs, off);
          };
          uint4 fr[3][2];
          rd(0, fr[0]);
          rd(1, fr[1]);
  #pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) rd(kk + 2, fr[(kk + 2) % 3]);
            // the reads go out before this step's MFMAs (the scheduler would
            // otherwise start the block's first MFMA after one read only)
            __builtin_amdgcn_sched_barrier(0);
            sacc = mfma32(as_bf16x8(fr[kk % 3][0]), as_bf16x8(qreg[kk]), sacc);
            pacc = mfma32(as_bf16x8(fr[kk % 3][1]), as_bf16x8(doreg[kk]), pacc);
            __builtin_amdgcn_sched_barrier(0);
          }
          // K^T operands of the dQ MFMAs go out now and land during the exponentials
          bf16x8 kt[CB][2];
  #pragma unroll
          for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
            for (int mm = 0; mm < 2; ++mm) kt[cb][mm] = a_from_rows_at<D>(ks, fo, 2 * blk + mm, cb);
          if (need_mask) {
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kt0 + blk * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
              if (key >= e || (causal && key > qi)) sacc[i] = -INFINITY;
            }
          }
          uint4 dsb[2];
  #pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            float ds[8];
  #pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int i = 8 * mm + j;
              ds[j] = fast_exp2(fmaf(sacc[i], a.sl2, -lse2)) * (pacc[i] + ndlt);
            }
            dsb[mm] = make_uint4(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                                 pack_bf16x2(ds[6], ds[7]));
          }
  #pragma unroll
          for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
            for (int mm = 0; mm < 2; ++mm)
              dqacc[cb] = mfma32(kt[cb][mm], as_bf16x8(dsb[mm]), dqacc[cb]);
        }
      }

      wait_vmem();
      __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, k0s, v0s, k1s, v1s);
      if (t + 1 < ntiles) step(t + 1, k1s, v1s, k0s, v0s);
    }
    tq.prefetch();  // the next tile's claim goes out before this one's stores

    if (qvalid) {
      bf16* out = a.dq + base + (size_t)qi * rs;
      if constexpr (kRing) {
        float* acc = a.dq_acc + base + (size_t)qi * rs;
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int c = cb * 32 + 8 * gq + 4 * half;
            add_store4(acc + c, dqacc[cb], 4 * gq, a.scale, rb.first, rb.last ? out + c : nullptr);
          }
      } else {
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<uint2*>(out + cb * 32 + 8 * gq + 4 * half) = pack4_scaled(dqacc[cb], 4 * gq, a.scale);
      }
    }
    tq.publish(s_claim);  // (its wait for the claim does not wait for the stores)
  }
  tq.finish();
}

// ------------------------------------------------------------------- dkdv kernel
// A workgroup owns 128 keys and walks 64-query tiles from the document end
// down to its first key (causal). Its 8 waves come in pairs that share a SIMD
// (waves p and p + 4) and 32 keys:
//   * producer p: K^T and V^T of the 32 keys stay in registers as B operands;
//     per tile it computes S = Q K^T and dP = dO V^T for both 32-query blocks
//     (lane = key), then P = exp2(S * log2(e) / sqrt(d) - lse2) and
//     dS = P (dP - D), packed to bf16 in the order the MFMA k index takes them
//     (query block 0's exponentials and packing run between block 1's MFMAs);
//   * consumers, one tile behind: consumer c accumulates dV^T += dO^T P and
//     dK^T += Q^T dS for the 64 keys of producers 2 (c/2) and 2 (c/2) + 1 and
//     half of the D columns, with the A operands read transposed from the
//     row-major Q and dO tiles (each serving both key blocks) and P, dS taken
//     from the producers through LDS (each serving both column blocks).
// The producer's exponentials run while the consumer keeps the SIMD's matrix
// core busy. Query tiles (Q, dO, lse2, D) arrive by direct-to-LDS loads one
// tile ahead, in three stages: the producer reads tile i while the consumer
// reads tile i - 1 and tile i + 1 lands. Two barriers per tile: after the
// first the producer overwrites the P/dS buffer the consumer has read, after
// the second the new P/dS and tile i + 1 are visible.
constexpr int kKvBK = 128;       // keys per workgroup
constexpr int kKvBQ = 64;        // queries per tile (two 32-query blocks)
constexpr int kKvThreads = 512;  // 4 producer and 4 consumer waves

template <int D>
struct KvStage {
  bf16 q[kKvBQ * D];     // RowTile layout
  bf16 dout[kKvBQ * D];  // RowTile layout
  float lse2[kKvBQ];
  float dlt[kKvBQ];  // -D
};

// Direct-to-LDS loads of one query tile: the 2 * kKvBQ rows of Q and dO are
// dealt to the 8 waves in 1 KB windows (waves 0-3 take Q, 4-7 dO); lane i
// lands on physical chunk i % (D/8) of its row and fetches the logical chunk
// the swizzle keeps there. Waves 0 and 1 also fetch lse2 and D, 4 bytes a
// lane. Buffer ranges end at the document end (zeros past it).
template <int D>
struct KvDma {
  static constexpr int CHUNKS = D / 8;
  static constexpr int ROWS_PER_OP = 64 / CHUNKS;
  static constexpr int OPS_PER_TENSOR = kKvBQ / ROWS_PER_OP;
  static constexpr int OPS = 2 * OPS_PER_TENSOR / (kKvThreads / 64);
  static_assert(OPS >= 1 && OPS * (kKvThreads / 64) == 2 * OPS_PER_TENSOR, "whole windows per wave");
  uint32_t voff[OPS];
  int lds_off[OPS];  // bf16 elements from the start of the tensor's tile
  bool is_dout;

  __device__ __forceinline__ void init(int w, int lane, uint32_t row_bytes) {
    is_dout = w >= (kKvThreads / 64) / 2;
#pragma unroll
    for (int j = 0; j < OPS; ++j) {
      const int op = (w * OPS + j) % OPS_PER_TENSOR;
      const int row0 = op * ROWS_PER_OP;
      const int r = row0 + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ RowTile<D>::chunk_key(r);
      voff[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16u;
      lds_off[j] = row0 * D;
    }
  }
  __device__ __forceinline__ void issue(rsrc_t rq, rsrc_t rd, rsrc_t rl, rsrc_t rdl, KvStage<D>& st, int w,
                                        int lane) const {
    const bf16* dst = is_dout ? st.dout : st.q;
    const rsrc_t src = is_dout ? rd : rq;
#pragma unroll
    for (int j = 0; j < OPS; ++j) buf_load16_lds(src, dst + lds_off[j], voff[j]);
    if (w == 0) buf_load4_lds(rl, st.lse2, (uint32_t)lane * 4u);
    if (w == 1) buf_load4_lds(rdl, st.dlt, (uint32_t)lane * 4u);
  }
};

// kRing: one ring step; row g = j * B + b holds key/value chunk j, its queries
// (Q, dO, lse, D) come from rank (j + step) mod sp, and dK, dV are added to
// dk_acc, dv_acc (written to dk, dv at the chunk's last step).
template <int D, bool kRing>
__global__ __launch_bounds__(kKvThreads, 1) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using L = RowTile<D>;
  constexpr int KK = D / 16;
  constexpr int CB = D / 32;
  // Three query-tile stages, separate arrays so that the compiler can tell a
  // stage being loaded from the stages being read.
  __shared__ __attribute__((aligned(16))) KvStage<D> st0;
  __shared__ __attribute__((aligned(16))) KvStage<D> st1;
  __shared__ __attribute__((aligned(16))) KvStage<D> st2;
  // P and dS of the last tile: per producer, per query block, 4 MFMA operands of 64 lanes
  __shared__ __attribute__((aligned(16))) uint4 xbuf[4 * 2 * 4 * 64];

  __shared__ int s_claim[4];
  TileQueue tq;
  tq.init(a.sched, a.nslots, a.ndoc, a.units);
  // The wave index is the same in every lane; saying so keeps the role
  // branches and the direct-to-LDS loads' LDS window (M0) scalar, where the
  // compiler would otherwise wrap each such load in a loop over the lanes'
  // distinct values (about 3% of this kernel's time).
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // One tile, for one role: producers and consumers run their own tile
  // loops (their registers stay apart) through the same sequence of barriers.
  auto tile = [&](const TileId& tid_, auto role) __attribute__((always_inline)) {
    constexpr bool producer = decltype(role)::value;
    const int lvl = tid_.lvl, doc = tid_.doc, unit = tid_.unit;
    int s, e;
    doc_range(a, doc, s, e);
    const int kb0 = s + lvl * kKvBK;  // causal: low key blocks have the most queries, so they go first
    if (kb0 >= e) return;             // the whole workgroup skips the tile

    const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
    const size_t rs = (size_t)a.Hl * D;
    const uint32_t row_bytes = (uint32_t)rs * 2u;
    const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
    size_t qbase = base;
    int qunit = unit;
    int causal = a.causal;
    RingBlock rb{g, a.causal, true, true};
    if constexpr (kRing) {
      if (!ring_block(a, g, false, rb)) return;  // the whole workgroup skips the tile
      causal = rb.causal;
      qbase = ((size_t)rb.other * a.N * a.Hl + hd) * D;
      qunit = rb.other * a.Hl + hd;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int pair = w & 3;
    const int kp0 = kb0 + 32 * pair;  // the pair's first key
    const int kj = kp0 + l32;         // this lane's key (producer waves)
    FragOffsets<D> fo;
    fo.init(lane);

    const int qstart = causal ? kb0 : s;
    const int ntiles = (e - qstart + kKvBQ - 1) / kKvBQ;
    // Query tiles are walked from the document end down: every workgroup of a
    // head then reads the same tile at about the same time, from the XCD's L2.
    const int qlast = qstart + (ntiles - 1) * kKvBQ;

    KvDma<D> dma;
    dma.init(w, lane, row_bytes);
    const float* lse2_u = a.lse2 + (size_t)qunit * a.N;
    const float* dl_u = a.delta + (size_t)qunit * a.N;
    auto load_tile = [&](int i, KvStage<D>& st) {
      const int qt0 = qlast - i * kKvBQ;
      const long long span = (long long)(e - qt0) * row_bytes;
      dma.issue(make_rsrc(a.q + qbase + (size_t)qt0 * rs, span), make_rsrc(a.dout + qbase + (size_t)qt0 * rs, span),
                make_rsrc(lse2_u + qt0, (long long)(e - qt0) * 4), make_rsrc(dl_u + qt0, (long long)(e - qt0) * 4),
                st, w, lane);
    };

    // The tile loop, with the three stages named per iteration (i mod 3):
    // work(i, cur, prev) runs between the loads of tile i + 1 going out and the
    // first barrier, publish(i) between the two barriers. Producers and
    // consumers run it with their own bodies, so that each role's registers are
    // its own; both pass the same barriers.
    auto tile_loop = [&](auto work, auto publish) {
      auto iteration = [&](int i, const KvStage<D>& cur, const KvStage<D>& prev, KvStage<D>& next) {
        if (i + 1 < ntiles) load_tile(i + 1, next);
        work(i, cur, prev);
        barrier_lds_only();  // the consumer has read the P/dS buffer
        publish(i);
        wait_vmem();
        __syncthreads();  // new P/dS and tile i + 1 visible
      };
      load_tile(0, st0);
      wait_vmem();
      __syncthreads();
      for (int i = 0; i <= ntiles; i += 3) {
        iteration(i, st0, st2, st1);
        if (i + 1 <= ntiles) iteration(i + 1, st1, st0, st2);
        if (i + 2 <= ntiles) iteration(i + 2, st2, st1, st0);
      }
    };

    if constexpr (producer) {
      // K^T and V^T of the pair's 32 keys (zero past the document end)
      uint4 kreg[KK], vreg[KK];
      {
        const long long span = (long long)(e - kp0) * row_bytes;
        const rsrc_t kr = make_rsrc(a.k + base + (size_t)kp0 * rs, span);
        const rsrc_t vr = make_rsrc(a.v + base + (size_t)kp0 * rs, span);
        const uint32_t off = (uint32_t)l32 * row_bytes + (uint32_t)(8 * half) * 2u;
  #pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kreg[kk] = buf_load16(kr, off + 32u * kk);
          vreg[kk] = buf_load16(vr, off + 32u * kk);
        }
      }
      // P and dS of both query blocks as MFMA B operands: pk[4 qb + mm] = P,
      // pk[4 qb + 2 + mm] = dS, accumulator elements 8 mm .. 8 mm + 7
      uint4 pk[8];
      auto produce = [&](int i, const KvStage<D>& st, const KvStage<D>&) {
        if (i >= ntiles) return;
        const int qt0 = qlast - i * kKvBQ;
        // tiles that cross the diagonal or a document end are masked element by element
        const bool need_mask = (causal && qt0 < kp0 + 31) || qt0 + kKvBQ > e || kp0 + 32 > e;
        // S = Q K^T and dP = dO V^T of both 32-query blocks. The exponentials of
        // block 0 run between the MFMAs of block 1, four elements every other
        // k-step (their lse2 and D read one step before), so the wave's own
        // matrix work covers half of its softmax.
        // dP starts from -D of its queries (the pre-pass stores D negated), so
        // the MFMAs leave dP - D and the softmax has no subtraction to do
        f32x16 sacc[2], pacc[2];
  #pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const float4 d4 = *reinterpret_cast<const float4*>(st.dlt + 32 * qb + 8 * gq + 4 * half);
            sacc[qb][4 * gq] = sacc[qb][4 * gq + 1] = sacc[qb][4 * gq + 2] = sacc[qb][4 * gq + 3] = 0.f;
            pacc[qb][4 * gq] = d4.x;
            pacc[qb][4 * gq + 1] = d4.y;
            pacc[qb][4 * gq + 2] = d4.z;
            pacc[qb][4 * gq + 3] = d4.w;
          }
        }
        // Q and dO fragments read two k-steps ahead of their MFMAs
        auto rd = [&](int qb, int kk, uint4* f) {
          const uint32_t off = fo.row_frag(qb, kk);
          f[0] = lds_ld16(st.q, off);
          f[1] = lds_ld16(st.dout, off);
        };
        // lse2 of the four queries of accumulator elements 4 gq .. 4 gq + 3
        auto rd_ld = [&](int qb, int gq, float4& l4) {
          l4 = *reinterpret_cast<const float4*>(st.lse2 + 32 * qb + 8 * gq + 4 * half);
        };
        // in place: sacc becomes P
        auto soft4 = [&](int qb, int gq, const float4& l4) {
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
  #pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int i2 = 4 * gq + x;
            sacc[qb][i2] = fast_exp2(fmaf(sacc[qb][i2], a.sl2, -lv[x]));
          }
        };
        // masked P (zero where the key is not visible to the query) and P (dP - D)
        // of accumulator elements 8 mm .. 8 mm + 7 of block qb, packed to bf16
        auto pack8 = [&](int qb, int mm) {
          const int b = 8 * mm;
          if (need_mask) {
  #pragma unroll
            for (int x = b; x < b + 8; ++x) {
              const int qq = qt0 + 32 * qb + 8 * (x >> 2) + 4 * half + (x & 3);
              if (qq >= e || kj >= e || (causal && kj > qq)) sacc[qb][x] = 0.f;
            }
          }
          const f32x16& p = sacc[qb];
          const f32x16& ds = pacc[qb];
          pk[4 * qb + mm] = make_uint4(pack_bf16x2(p[b], p[b + 1]), pack_bf16x2(p[b + 2], p[b + 3]),
                                       pack_bf16x2(p[b + 4], p[b + 5]), pack_bf16x2(p[b + 6], p[b + 7]));
          pk[4 * qb + 2 + mm] = make_uint4(pack_bf16x2(p[b] * ds[b], p[b + 1] * ds[b + 1]),
                                           pack_bf16x2(p[b + 2] * ds[b + 2], p[b + 3] * ds[b + 3]),
                                           pack_bf16x2(p[b + 4] * ds[b + 4], p[b + 5] * ds[b + 5]),
                                           pack_bf16x2(p[b + 6] * ds[b + 6], p[b + 7] * ds[b + 7]));
        };
        {
          uint4 fr[3][2];
          rd(0, 0, fr[0]);
          rd(0, 1, fr[1]);
  #pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) rd(0, kk + 2, fr[(kk + 2) % 3]);
            sacc[0] = mfma32(as_bf16x8(fr[kk % 3][0]), as_bf16x8(kreg[kk]), sacc[0]);
            pacc[0] = mfma32(as_bf16x8(fr[kk % 3][1]), as_bf16x8(vreg[kk]), pacc[0]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        {
          uint4 fr[3][2];
          float4 l4;
          rd(1, 0, fr[0]);
          rd(1, 1, fr[1]);
  #pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + 2 < KK) rd(1, kk + 2, fr[(kk + 2) % 3]);
            if ((kk & 1) == 0 && kk / 2 < 4) rd_ld(0, kk / 2, l4);
            sacc[1] = mfma32(as_bf16x8(fr[kk % 3][0]), as_bf16x8(kreg[kk]), sacc[1]);
            pacc[1] = mfma32(as_bf16x8(fr[kk % 3][1]), as_bf16x8(vreg[kk]), pacc[1]);
            if ((kk & 1) == 1 && kk / 2 < 4) soft4(0, kk / 2, l4);
            if (kk == 3 || kk == 7) pack8(0, kk / 4);
            __builtin_amdgcn_sched_barrier(0);
          }
          // with D = 64 there are only four k-steps: the rest of block 0 here
  #pragma unroll
          for (int gq = KK / 2; gq < 4; ++gq) {
            rd_ld(0, gq, l4);
            soft4(0, gq, l4);
          }
          if (KK < 8) pack8(0, 1);
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            rd_ld(1, gq, l4);
            soft4(1, gq, l4);
          }
        }
  #pragma unroll
        for (int mm = 0; mm < 2; ++mm) pack8(1, mm);
      };
      auto publish = [&](int i) {
        if (i >= ntiles) return;
  #pragma unroll
        for (int qb = 0; qb < 2; ++qb)
  #pragma unroll
          for (int j = 0; j < 4; ++j) xbuf[((pair * 2 + qb) * 4 + j) * 64 + lane] = pk[4 * qb + j];
      };
      tile_loop(produce, publish);
    } else {
      // Consumer c takes the P/dS of producer pairs 2 (c/2) and 2 (c/2) + 1 (64
      // keys) and accumulates dK^T, dV^T for half of the D columns, those of
      // column blocks CH (c % 2) .. CH (c % 2) + CH - 1: every A fragment (dO^T,
      // Q^T) it reads serves both key blocks and every P/dS operand both column
      // blocks.
      constexpr int CH = CB / 2;
      const int kp_first = 2 * (pair >> 1);  // first producer pair of this consumer
      const int cb0 = CH * (pair & 1);
      f32x16 dkacc[2][CH], dvacc[2][CH];  // [key block][column block]
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
        for (int c = 0; c < CH; ++c)
  #pragma unroll
          for (int i = 0; i < 16; ++i) dkacc[kb][c][i] = dvacc[kb][c][i] = 0.f;
      // the previous tile, in four steps (query block qb, 16-query half hf):
      // A = dO^T, Q^T of those 16 queries for the CH column blocks, B = P, dS
      // of the two key blocks; the next step's operands are read while this
      // step's MFMAs run
      auto consume = [&](int i, const KvStage<D>&, const KvStage<D>& st) {
        if (i < 1) return;
        auto rd = [&](int step, bf16x8 (*fa)[2], uint4 (*fb)[2]) {
          const int qb = step >> 1, hf = step & 1;
  #pragma unroll
          for (int c = 0; c < CH; ++c) {
            fa[c][0] = a_from_rows_at<D>(st.dout, fo, 2 * qb + hf, cb0 + c);
            fa[c][1] = a_from_rows_at<D>(st.q, fo, 2 * qb + hf, cb0 + c);
          }
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            fb[kb][0] = xbuf[(((kp_first + kb) * 2 + qb) * 4 + hf) * 64 + lane];
            fb[kb][1] = xbuf[(((kp_first + kb) * 2 + qb) * 4 + 2 + hf) * 64 + lane];
          }
        };
        bf16x8 fa[2][CH][2];
        uint4 fb[2][2][2];
        rd(0, fa[0], fb[0]);
  #pragma unroll
        for (int step = 0; step < 4; ++step) {
          if (step + 1 < 4) rd(step + 1, fa[(step + 1) & 1], fb[(step + 1) & 1]);
          const int cur = step & 1;
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
            for (int c = 0; c < CH; ++c) {
              dvacc[kb][c] = mfma32(fa[cur][c][0], as_bf16x8(fb[cur][kb][0]), dvacc[kb][c]);
              dkacc[kb][c] = mfma32(fa[cur][c][1], as_bf16x8(fb[cur][kb][1]), dkacc[kb][c]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      tile_loop(consume, [](int) {});

  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kc = kb0 + 32 * (kp_first + kb) + l32;  // this lane's key in key block kb
        if (kc < e) {
          bf16* ko = a.dk + base + (size_t)kc * rs;
          bf16* vo = a.dv + base + (size_t)kc * rs;
          if constexpr (kRing) {
            float* ka = a.dk_acc + base + (size_t)kc * rs;
            float* va = a.dv_acc + base + (size_t)kc * rs;
  #pragma unroll
            for (int c = 0; c < CH; ++c)
  #pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const int col = 32 * (cb0 + c) + 8 * gq + 4 * half;
                add_store4(ka + col, dkacc[kb][c], 4 * gq, a.scale, rb.first, rb.last ? ko + col : nullptr);
                add_store4(va + col, dvacc[kb][c], 4 * gq, 1.f, rb.first, rb.last ? vo + col : nullptr);
              }
          } else {
  #pragma unroll
            for (int c = 0; c < CH; ++c)
  #pragma unroll
              for (int gq = 0; gq < 4; ++gq) {
                const int col = 32 * (cb0 + c) + 8 * gq + 4 * half;
                *reinterpret_cast<uint2*>(ko + col) = pack4_scaled(dkacc[kb][c], 4 * gq, a.scale);
                *reinterpret_cast<uint2*>(vo + col) = pack4_scaled(dvacc[kb][c], 4 * gq, 1.f);
              }
          }
        }
      }
    }
  };
  TileId t;
  if (w < 4) {
    while (tq.next(t, s_claim)) tile(t, RoleTag<true>{});
  } else {
    while (tq.next(t, s_claim)) tile(t, RoleTag<false>{});
  }
  tq.finish();
}

}  // namespace

namespace uly_host {

int device_cu_count() {
  static std::mutex mu;
  static int cache[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// The queue counters behind the 2 * rows floats of a backward workspace
// (256-byte aligned offset; ulysses_attn_bwd_workspace_bytes counts them).
constexpr size_t kSchedBytes = 2 * uly::kQueueBytes;
inline size_t sched_offset(size_t rows) { return (2 * rows * sizeof(float) + 255) / 256 * 256; }
int* sched_counters(float* ws, size_t rows) {
  return reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + sched_offset(rows));
}
size_t bwd_workspace_bytes(size_t rows) { return sched_offset(rows) + kSchedBytes; }

// The tile decode forms nslots * ndoc * max(units, kUnitGroup) in int, for
// the dQ kernel's 256-query tiles and the dK/dV kernel's 128-key tiles.
bool bwd_tiles_fit(const AttnGeom& g) {
  const long long maxlen = g.cu ? g.max_doc_len : g.N;
  const long long units = (long long)g.G * g.Hl;
  const long long ug = units > uly::kUnitGroup ? units : uly::kUnitGroup;
  return (maxlen + kKvBK - 1) / kKvBK * g.ndoc * ug <= 0x7fffffffLL &&
         (maxlen + kDqBQ - 1) / kDqBQ * g.ndoc * ug <= 0x7fffffffLL;
}

int launch_attn_bwd_main_bf16(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, const float* delta,
                              const AttnGeom& g, void* stream) {
  if (!bwd_tiles_fit(g)) return ULY_ESHAPE;
  BwdArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = nullptr;
  a.dout = static_cast<const bf16*>(dout);
  a.lse = lse;
  a.delta = const_cast<float*>(delta);
  a.lse2 = const_cast<float*>(delta) + (size_t)g.G * g.Hl * g.N;
  a.dq = static_cast<bf16*>(dq);
  a.dk = static_cast<bf16*>(dk);
  a.dv = static_cast<bf16*>(dv);
  a.cu = g.cu;
  a.ndoc = g.ndoc;
  a.units = g.G * g.Hl;
  a.Hl = g.Hl;
  a.N = g.N;
  a.causal = g.causal;
  a.scale = 1.0f / sqrtf((float)g.d);
  a.sl2 = uly::kLog2e * a.scale;
  a.dq_acc = a.dk_acc = a.dv_acc = nullptr;
  a.step = 0;
  a.sp = 1;
  a.B = 1;
  a.sched = nullptr;
  const int maxlen = g.cu ? g.max_doc_len : g.N;
  hipStream_t st = (hipStream_t)stream;

  BwdArgs aq = a;
  aq.nslots = (maxlen + kDqBQ - 1) / kDqBQ;
  const long long qblocks = (long long)aq.nslots * a.ndoc * a.units;
  BwdArgs akv = a;
  akv.nslots = (maxlen + kKvBK - 1) / kKvBK;
  const long long kvblocks = (long long)akv.nslots * a.ndoc * a.units;

  // Persistent launches: one workgroup per compute unit (each kernel holds a
  // whole CU), taking tiles from the queues in the workspace's tail, which
  // the pre-pass cleared and each kernel leaves cleared.
  const int ncu = device_cu_count();
  int* sched = sched_counters(const_cast<float*>(delta), (size_t)g.G * g.Hl * g.N);
  long long kvgrid = kvblocks, qgrid = qblocks;
  if (ncu > 0) {
    akv.sched = sched;
    aq.sched = sched + kSchedDq;
    kvgrid = kvblocks < ncu ? kvblocks : ncu;
    qgrid = qblocks < ncu ? qblocks : ncu;
  }
  if (g.d == 64) {
    hipLaunchKernelGGL((attn_dkdv_bf16_kernel<64, false>), dim3((unsigned)kvgrid), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL((attn_dq_bf16_kernel<64, false>), dim3((unsigned)qgrid), dim3(kDqThreads), 0, st, aq);
  } else {
    hipLaunchKernelGGL((attn_dkdv_bf16_kernel<128, false>), dim3((unsigned)kvgrid), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL((attn_dq_bf16_kernel<128, false>), dim3((unsigned)qgrid), dim3(kDqThreads), 0, st, aq);
  }
  return launch_status();
}

int launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, const AttnGeom& g, void* stream) {
  if (!bwd_tiles_fit(g)) return ULY_ESHAPE;  // before the pre-pass is enqueued
  const int rc = launch_attn_bwd_prepare_bf16(o, dout, lse, delta, g, stream, true);
  if (rc != ULY_OK) return rc;
  return launch_attn_bwd_main_bf16(q, k, v, dout, lse, dq, dk, dv, delta, g, stream);
}

// The D pre-pass over G rows of N tokens and Hl heads: -D and lse * log2(e)
// into the workspace (Ulysses shares and ring chunks alike).
int launch_attn_bwd_prepare_bf16(const void* o, const void* dout, const float* lse, float* delta,
                                 const AttnGeom& g, void* stream, bool with_sched) {
  const long long rows = (long long)g.G * g.Hl * g.N;
  const long long units = (long long)g.G * g.Hl;
  const int tpb = kDeltaPasses * kThreads / (g.d / 8);  // tokens per block
  const dim3 dgrid((unsigned)((g.N + tpb - 1) / tpb), (unsigned)(units < 65535 ? units : 65535));
  const bf16* ob = static_cast<const bf16*>(o);
  const bf16* db = static_cast<const bf16*>(dout);
  float* lse2 = delta + (size_t)rows;
  int* sched = with_sched ? sched_counters(delta, (size_t)rows) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (g.d == 64)
    hipLaunchKernelGGL(delta_bf16_kernel<64>, dgrid, dim3(kThreads), 0, st, ob, db, lse, delta,
                       lse2, g.N, g.Hl, units, sched);
  else
    hipLaunchKernelGGL(delta_bf16_kernel<128>, dgrid, dim3(kThreads), 0, st, ob, db, lse, delta,
                       lse2, g.N, g.Hl, units, sched);
  return launch_status();
}

int launch_ring_bwd_bf16(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         float* delta, float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk,
                         void* dv, const AttnGeom& g, int sp, int B, int step, void* stream) {
  BwdArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = nullptr;
  a.dout = static_cast<const bf16*>(dout);
  a.lse = lse;
  a.delta = const_cast<float*>(delta);
  a.lse2 = const_cast<float*>(delta) + (size_t)g.G * g.Hl * g.N;
  a.dq = static_cast<bf16*>(dq);
  a.dk = static_cast<bf16*>(dk);
  a.dv = static_cast<bf16*>(dv);
  a.cu = nullptr;
  a.ndoc = 1;
  a.units = g.G * g.Hl;
  a.Hl = g.Hl;
  a.N = g.N;
  a.causal = g.causal;
  a.scale = 1.0f / sqrtf((float)g.d);
  a.sl2 = uly::kLog2e * a.scale;
  a.dq_acc = dq_acc;
  a.dk_acc = dk_acc;
  a.dv_acc = dv_acc;
  a.step = step;
  a.sp = sp;
  a.B = B;
  a.sched = nullptr;
  BwdArgs aq = a;
  aq.nslots = (g.N + kDqBQ - 1) / kDqBQ;
  BwdArgs akv = a;
  akv.nslots = (g.N + kKvBK - 1) / kKvBK;
  const long long qblocks = (long long)aq.nslots * a.units;
  const long long kvblocks = (long long)akv.nslots * a.units;
  const long long ug = a.units > uly::kUnitGroup ? a.units : uly::kUnitGroup;
  if ((long long)aq.nslots * ug > 0x7fffffffLL || (long long)akv.nslots * ug > 0x7fffffffLL) return ULY_ESHAPE;
  // Persistent launches, as in the Ulysses backward: the queue counters sit in
  // the workspace's tail (the prepare call cleared them, each kernel leaves
  // them cleared for the next step); tiles of rows whose chunk this step does
  // not reach are claimed and passed over.
  const int ncu = device_cu_count();
  long long kvgrid = kvblocks, qgrid = qblocks;
  if (ncu > 0) {
    int* sched = sched_counters(delta, (size_t)g.G * g.Hl * g.N);
    akv.sched = sched;
    aq.sched = sched + kSchedDq;
    kvgrid = kvblocks < ncu ? kvblocks : ncu;
    qgrid = qblocks < ncu ? qblocks : ncu;
  }
  hipStream_t st = (hipStream_t)stream;
  if (g.d == 64) {
    hipLaunchKernelGGL((attn_dkdv_bf16_kernel<64, true>), dim3((unsigned)kvgrid), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL((attn_dq_bf16_kernel<64, true>), dim3((unsigned)qgrid), dim3(kDqThreads), 0, st, aq);
  } else {
    hipLaunchKernelGGL((attn_dkdv_bf16_kernel<128, true>), dim3((unsigned)kvgrid), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL((attn_dq_bf16_kernel<128, true>), dim3((unsigned)qgrid), dim3(kDqThreads), 0, st, aq);
  }
  return launch_status();
}

}  // namespace uly_host

extern "C" size_t ulysses_attn_bwd_workspace_bytes(int sp, int B, int N, int Hl, int d, int dtype) {
  if (sp <= 0 || B <= 0 || N <= 0 || Hl <= 0) return 0;
  if (!uly_host::dtype_ok(dtype) || !uly_host::head_dim_ok(d)) return 0;
  // -D = -rowsum(dO * O) and lse in log2 units: two floats per (rank, batch row, head, token),
  // then the tile-queue counters of the dK/dV and dQ kernels.
  return uly_host::bwd_workspace_bytes((size_t)sp * B * Hl * N);
}

extern "C" int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, const int* cu_seqlens,
                                int ndoc, int max_doc_len, int sp, int B, int N, int Hl, int d,
                                int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ULY_EINVAL;
  const int rc = uly_host::check_attn_args(ndoc, max_doc_len, cu_seqlens, sp, B, N, Hl, d, dtype);
  if (rc != ULY_OK) return rc;
  const size_t need = ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, dtype);
  if (!workspace || workspace_bytes < need) return ULY_EWORKSPACE;
  uly_host::AttnGeom g;
  g.G = sp * B;
  g.N = N;
  g.Hl = Hl;
  g.d = d;
  g.cu = cu_seqlens;
  g.ndoc = cu_seqlens ? ndoc : 1;
  g.max_doc_len = cu_seqlens ? max_doc_len : N;
  g.causal = causal ? 1 : 0;
  float* delta = static_cast<float*>(workspace);
  if (dtype == ULY_F32)
    return uly_host::launch_attn_bwd_f32(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(o), static_cast<const float*>(dout), lse, static_cast<float*>(dq),
        static_cast<float*>(dk), static_cast<float*>(dv), delta, g, stream);
  return uly_host::launch_attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, g, stream);
}

namespace {

// Host checks of the split backward's calls; fills the geometry.
int bwd_split_args(const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B, int N, int Hl, int d,
                   int causal, int dtype, size_t workspace_bytes, const void* workspace, uly_host::AttnGeom& g) {
  const int rc = uly_host::check_attn_args(ndoc, max_doc_len, cu_seqlens, sp, B, N, Hl, d, dtype);
  if (rc != ULY_OK) return rc;
  if (!workspace || workspace_bytes < ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, dtype)) return ULY_EWORKSPACE;
  g.G = sp * B;
  g.N = N;
  g.Hl = Hl;
  g.d = d;
  g.cu = cu_seqlens;
  g.ndoc = cu_seqlens ? ndoc : 1;
  g.max_doc_len = cu_seqlens ? max_doc_len : N;
  g.causal = causal ? 1 : 0;
  return ULY_OK;
}

}  // namespace

extern "C" int ulysses_attn_bwd_prepare(const void* o, const void* dout, const float* lse, void* workspace,
                                        size_t workspace_bytes, int sp, int B, int N, int Hl, int d, int dtype,
                                        void* stream) {
  if (!o || !dout || !lse) return ULY_EINVAL;
  uly_host::AttnGeom g;
  const int rc = bwd_split_args(nullptr, 1, N, sp, B, N, Hl, d, 1, dtype, workspace_bytes, workspace, g);
  if (rc != ULY_OK) return rc;
  float* delta = static_cast<float*>(workspace);
  if (dtype == ULY_F32)
    return uly_host::launch_attn_bwd_prepare_f32(static_cast<const float*>(o), static_cast<const float*>(dout),
                                                 delta, g, stream);
  return uly_host::launch_attn_bwd_prepare_bf16(o, dout, lse, delta, g, stream, true);
}

extern "C" int ulysses_attn_bwd_prepared(const void* q, const void* k, const void* v, const void* dout,
                                         const float* lse, void* dq, void* dk, void* dv, void* workspace,
                                         size_t workspace_bytes, const int* cu_seqlens, int ndoc, int max_doc_len,
                                         int sp, int B, int N, int Hl, int d, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv) return ULY_EINVAL;
  uly_host::AttnGeom g;
  const int rc = bwd_split_args(cu_seqlens, ndoc, max_doc_len, sp, B, N, Hl, d, causal, dtype, workspace_bytes,
                                workspace, g);
  if (rc != ULY_OK) return rc;
  const float* delta = static_cast<const float*>(workspace);
  if (dtype == ULY_F32)
    return uly_host::launch_attn_bwd_main_f32(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(dout), lse, static_cast<float*>(dq), static_cast<float*>(dk),
        static_cast<float*>(dv), delta, g, stream);
  return uly_host::launch_attn_bwd_main_bf16(q, k, v, dout, lse, dq, dk, dv, delta, g, stream);
}

// ----------------------------------------------------- no-allocation variant
// ulysses_attn_bwd_noalloc keeps what the workspace of ulysses_attn_bwd holds
// (-D and lse in log2 units, two floats per row) in this file-scope array
// instead: one copy on every GPU the library runs on, from the module's load
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory, so the kernels are given the device address looked up
// once per device with hipGetSymbolAddress.
static_assert(ULY_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) float scratch[ULY_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices];  // device address of `scratch` on device i, once looked up

// The scratch address on the calling thread's current device.
int current_device_scratch(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ULY_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ULY_EHIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return ULY_OK;
}

}  // namespace

extern "C" int ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                        const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B,
                                        int N, int Hl, int d, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ULY_EINVAL;
  const int rc = uly_host::check_attn_args(ndoc, max_doc_len, cu_seqlens, sp, B, N, Hl, d, dtype);
  if (rc != ULY_OK) return rc;
  const size_t need = ulysses_attn_bwd_workspace_bytes(sp, B, N, Hl, d, dtype);
  if (need > ULY_NOALLOC_SCRATCH_BYTES) return ULY_EWORKSPACE;
  float* ws = nullptr;
  const int src = current_device_scratch(&ws);
  if (src != ULY_OK) return src;
  return ulysses_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, need, cu_seqlens, ndoc, max_doc_len, sp, B,
                          N, Hl, d, causal, dtype, stream);
}
