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
//   * dq kernel, query-stationary: a workgroup owns 128 queries (32 per
//     wave, Q and dO resident in registers as MFMA B operands) and walks the
//     64-key K/V tiles of its document (double-buffered in LDS). Per tile: S^T = K Q^T and
//     dP^T = V dO^T (lane = query, so lse_i and D_i are per-lane scalars),
//     dS^T in registers, then dQ^T += K^T dS^T (K^T read from the row-major
//     K tile with gfx950's transposing LDS reads).
//   * dkdv kernel, key-stationary: a workgroup of 8 waves owns 128 keys (K
//     and V resident as B operands, each 32-key group shared by two waves)
//     and walks 64-query tiles (Q, dO, lse, D double-buffered in LDS) from the
//     document end down to its first key (causal). Per tile: S = Q K^T and dP = dO V^T
//     (lane = key), then dV^T += dO^T P and dK^T += Q^T dS with the A
//     operands read transposed from the row-major Q and dO tiles; the
//     accumulators hold one key per lane, so the final stores are 4
//     consecutive columns per lane.
// The MFMA k index of a 16-wide step maps to tokens the same way as in the
// forward kernel, so P and dS feed the MFMA straight from the accumulators.

#include <math.h>

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
  float* delta;
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
};

__device__ __forceinline__ void doc_range(const BwdArgs& a, int doc, int& s, int& e) {
  s = 0;
  e = a.N;
  if (a.cu) {
    s = a.cu[doc];
    e = a.cu[doc + 1];
  }
}

// ------------------------------------------------------------------ D pre-pass
// D[unit][t] = sum_c dO[t][c] * O[t][c]; D/8 lanes per row, 16 bytes per lane.
template <int D>
__global__ __launch_bounds__(kThreads) void delta_bf16_kernel(const bf16* __restrict__ o,
                                                              const bf16* __restrict__ dout,
                                                              float* __restrict__ delta, int N, int Hl,
                                                              long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = kThreads / LPR;
  const int sub = threadIdx.x % LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  float acc = 0.f;
  if (row < rows) {
    // row enumerates (unit, t) with t fastest; unit = g * Hl + h
    const long long unit = row / N;
    const int t = (int)(row - unit * N);
    const long long g = unit / Hl;
    const int h = (int)(unit - g * Hl);
    const size_t off = ((size_t)(g * N + t) * Hl + h) * D + sub * 8;
    const uint4 ov = *reinterpret_cast<const uint4*>(o + off);
    const uint4 dv = *reinterpret_cast<const uint4*>(dout + off);
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov);
    const uint32_t* dw = reinterpret_cast<const uint32_t*>(&dv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_bits_to_float(ow[j] & 0xffffu), bf16_bits_to_float(dw[j] & 0xffffu), acc);
      acc = fmaf(bf16_bits_to_float(ow[j] >> 16), bf16_bits_to_float(dw[j] >> 16), acc);
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && sub == 0) delta[row] = acc;
}

// ----------------------------------------------------------- shared tile staging
// A tile of kRows tokens of two [token][d] tensors, staged global -> registers
// -> LDS (RowTile layout) by kNT threads. Thread tid moves the 16-byte chunks
// id = tid + j*kNT (token id/(D/8), column chunk id%(D/8)). Loads go
// through buffer resources ending at the document end: rows past it read as
// zero and the per-thread offsets are the same for every tile.
template <int D, int kRows, int kNT = kThreads>
struct PairTile {
  using L = RowTile<D>;
  static constexpr int RS = L::RS;                  // LDS row stride (bf16)
  static constexpr int CH = kRows * D / 8 / kNT;    // chunks per thread per tensor
  static constexpr int kRowStep = kNT / (D / 8);    // tokens between a thread's chunks
  uint4 a[CH];
  uint4 b[CH];

  __device__ __forceinline__ void load(rsrc_t ra, rsrc_t rb, uint32_t off0, uint32_t row_bytes) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t off = off0 + (uint32_t)(j * kRowStep) * row_bytes;
      a[j] = buf_load16(ra, off);
      b[j] = buf_load16(rb, off);
    }
  }
  __device__ __forceinline__ void store(bf16* sa, bf16* sb, int tid) const {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int at = L::off(tid / (D / 8) + j * kRowStep, (tid % (D / 8)) * 8);
      *reinterpret_cast<uint4*>(sa + at) = a[j];
      *reinterpret_cast<uint4*>(sb + at) = b[j];
    }
  }
};

// --------------------------------------------------------------------- dq kernel
constexpr int kDqBQ = 128;  // queries per workgroup (32 per wave)
constexpr int kDqBK = 64;   // keys per tile

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_dq_bf16_kernel(BwdArgs a) {
  using T = PairTile<D, kDqBK>;
  constexpr int RS = T::RS;
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int TILE = kDqBK * RS;   // bf16 elements of one staged tensor
  constexpr int STAGE = 2 * TILE;    // K then V
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int per_level = a.ndoc * a.units;
  const int lvl = blockIdx.x / per_level;
  const int rem = blockIdx.x - lvl * per_level;
  const int doc = rem / a.units;
  const int unit = rem - doc * a.units;
  int s, e;
  doc_range(a, doc, s, e);
  const int q0 = s + (a.nslots - 1 - lvl) * kDqBQ;
  if (q0 >= e) return;  // the whole workgroup leaves before any barrier

  const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
  const size_t rs = (size_t)a.Hl * D;
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int qi = q0 + 32 * w + l32;
  const bool qvalid = qi < e;

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
  const float dlt = qvalid ? a.delta[(size_t)unit * a.N + qi] : 0.f;

  const int kend = a.causal ? min(e, q0 + kDqBQ) : e;
  const int ntiles = (kend - s + kDqBK - 1) / kDqBK;

  f32x16 dqacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[cb][i] = 0.f;

  const uint32_t off0 = (uint32_t)(tid / (D / 8)) * row_bytes + (uint32_t)(tid % (D / 8)) * 16u;
  auto rsrc_at = [&](const bf16* p, int kt0) {
    return make_rsrc(p + base + (size_t)kt0 * rs, (long long)(e - kt0) * row_bytes);
  };
  T tile;
  tile.load(rsrc_at(a.k, s), rsrc_at(a.v, s), off0, row_bytes);
  tile.store(smem, smem + TILE, tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = s + t * kDqBK;
    const bf16* ks = smem + (t & 1) * STAGE;
    const bf16* vs = ks + TILE;
    const bool more = t + 1 < ntiles;
    if (more) tile.load(rsrc_at(a.k, kt0 + kDqBK), rsrc_at(a.v, kt0 + kDqBK), off0, row_bytes);

    if (!a.causal || kt0 <= q0 + 32 * w + 31) {
      const bool need_mask = (a.causal && kt0 + kDqBK - 1 > q0) || kt0 + kDqBK > e;
      // one 32-key block at a time: S^T = K Q^T and dP^T = V dO^T (lane = query,
      // element i is key kt0 + blk*32 + 8*(i/4) + 4*half + (i%4)), dS^T, then
      // dQ^T += K^T dS^T with K^T read from the K tile by transposing reads
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int off = T::L::off(blk * 32 + l32, 16 * kk + 8 * half);
          const uint4 ka = *reinterpret_cast<const uint4*>(ks + off);
          const uint4 va = *reinterpret_cast<const uint4*>(vs + off);
          sacc = mfma32(as_bf16x8(ka), as_bf16x8(qreg[kk]), sacc);
          pacc = mfma32(as_bf16x8(va), as_bf16x8(doreg[kk]), pacc);
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt0 + blk * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key >= e || (a.causal && key > qi)) sacc[i] = -INFINITY;
          }
        }
        uint4 dsb[2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * mm + j;
            ds[j] = fast_exp2(fmaf(sacc[i], a.sl2, -lse2)) * (pacc[i] - dlt);
          }
          dsb[mm] = make_uint4(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]), pack_bf16x2(ds[4], ds[5]),
                               pack_bf16x2(ds[6], ds[7]));
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
            dqacc[cb] = mfma32(a_from_rows<D>(ks, 32 * blk + 16 * mm, 32 * cb, lane), as_bf16x8(dsb[mm]), dqacc[cb]);
      }
    }

    if (more) {
      bf16* nk = smem + ((t + 1) & 1) * STAGE;
      tile.store(nk, nk + TILE, tid);
    }
    __syncthreads();
  }

  if (qvalid) {
    bf16* out = a.dq + base + (size_t)qi * rs;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        *reinterpret_cast<uint2*>(out + cb * 32 + 8 * gq + 4 * half) = pack4_scaled(dqacc[cb], 4 * gq, a.scale);
  }
}

// ------------------------------------------------------------------- dkdv kernel
// 8 waves, 128 keys per workgroup. Waves w and w + 4 share the 32 keys
// kb0 + 32*(w % 4): each computes S, dP, P and dS for one of the tile's two
// 32-query blocks (block w / 4), hands its packed P and dS to the other wave
// through LDS, and accumulates dK and dV for one half of the head dimension
// (columns [w/4 * D/2, w/4 * D/2 + D/2)) over both blocks. No MFMA is done
// twice, and with half the accumulators per wave two waves fit on a SIMD.
constexpr int kKvBK = 128;      // keys per workgroup
constexpr int kKvBQ = 64;       // queries per tile (two 32-query blocks)
constexpr int kKvThreads = 512; // 8 waves

template <int D>
__global__ __launch_bounds__(kKvThreads, 1) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using T = PairTile<D, kKvBQ, kKvThreads>;
  constexpr int KK = D / 16;
  constexpr int CBH = D / 64;                 // 32-column blocks per wave (half of D / 32)
  constexpr int TILE = kKvBQ * T::RS;         // bf16 elements of one staged tensor
  constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * kKvBQ * 4;  // Q, dO, then lse (log2 units) and D
  constexpr int XCH_BYTES = 8 * 4 * 64 * 16;  // per wave: P and dS as 4 x 16 bytes per lane
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * STAGE_BYTES + XCH_BYTES];
  uint4* xch = reinterpret_cast<uint4*>(smem_raw + 2 * STAGE_BYTES);

  const int per_level = a.ndoc * a.units;
  const int lvl = blockIdx.x / per_level;
  const int rem = blockIdx.x - lvl * per_level;
  const int doc = rem / a.units;
  const int unit = rem - doc * a.units;
  int s, e;
  doc_range(a, doc, s, e);
  const int kb0 = s + lvl * kKvBK;  // causal: low key blocks have the most queries, so they go first
  if (kb0 >= e) return;             // the whole workgroup leaves before any barrier

  const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
  const size_t rs = (size_t)a.Hl * D;
  const uint32_t row_bytes = (uint32_t)rs * 2u;
  const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int kgrp = w & 3, role = w >> 2;  // key group; query block and column half of this wave
  const int kj = kb0 + 32 * kgrp + l32;

  // K^T and V^T of the wave's 32 keys as resident B operands (zero past the document end)
  uint4 kreg[KK], vreg[KK];
  {
    const long long span = (long long)(e - kb0) * row_bytes;
    const rsrc_t kr = make_rsrc(a.k + base + (size_t)kb0 * rs, span);
    const rsrc_t vr = make_rsrc(a.v + base + (size_t)kb0 * rs, span);
    const uint32_t off = (uint32_t)(32 * kgrp + l32) * row_bytes + (uint32_t)(8 * half) * 2u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kreg[kk] = buf_load16(kr, off + 32u * kk);
      vreg[kk] = buf_load16(vr, off + 32u * kk);
    }
  }

  const int qstart = a.causal ? kb0 : s;
  const int ntiles = (e - qstart + kKvBQ - 1) / kKvBQ;
  const float* lse_u = a.lse + (size_t)unit * a.N;
  const float* dl_u = a.delta + (size_t)unit * a.N;

  f32x16 dkacc[CBH], dvacc[CBH];
#pragma unroll
  for (int c = 0; c < CBH; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[c][i] = dvacc[c][i] = 0.f;

  // staging: Q and dO chunks; threads [0, 64) also carry the tile's lse (log2
  // units), threads [64, 128) its D
  const uint32_t off0 = (uint32_t)(tid / (D / 8)) * row_bytes + (uint32_t)(tid % (D / 8)) * 16u;
  T tile;
  float sv = 0.f;
  auto load = [&](int qt0) {
    const long long span = (long long)(e - qt0) * row_bytes;
    tile.load(make_rsrc(a.q + base + (size_t)qt0 * rs, span), make_rsrc(a.dout + base + (size_t)qt0 * rs, span),
              off0, row_bytes);
    if (tid < 2 * kKvBQ) {
      const int qq = qt0 + (tid % kKvBQ);
      if (tid < kKvBQ) sv = qq < e ? lse_u[qq] * kLog2e : 0.f;
      else sv = qq < e ? dl_u[qq] : 0.f;
    }
  };
  auto store = [&](uint8_t* stage) {
    bf16* sm = reinterpret_cast<bf16*>(stage);
    tile.store(sm, sm + TILE, tid);
    if (tid < 2 * kKvBQ) reinterpret_cast<float*>(stage + 2 * TILE * 2)[tid] = sv;
  };

  // Query tiles are walked from the document end down to the first one this
  // block needs: every workgroup of a head then reads the same Q/dO tile at
  // about the same time, so the XCD's L2 serves them all.
  const int qlast = qstart + (ntiles - 1) * kKvBQ;
  load(qlast);
  store(smem_raw);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int qt0 = qlast - t * kKvBQ;
    const uint8_t* stage = smem_raw + (t & 1) * STAGE_BYTES;
    const bf16* qs = reinterpret_cast<const bf16*>(stage);
    const bf16* dos = qs + TILE;
    const float* sf = reinterpret_cast<const float*>(stage + 2 * TILE * 2);
    const bool more = t + 1 < ntiles;
    if (more) load(qt0 - kKvBQ);

    // ---- this wave's query block: S = Q K^T, dP = dO V^T (lane = key kj,
    // element i is query qb0 + 8*(i/4) + 4*half + (i%4)), then P and dS
    const int qb0 = qt0 + 32 * role;
    f32x16 sacc, pacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int off = RowTile<D>::off(32 * role + l32, 16 * kk + 8 * half);
      const uint4 qa = *reinterpret_cast<const uint4*>(qs + off);
      const uint4 da = *reinterpret_cast<const uint4*>(dos + off);
      sacc = mfma32(as_bf16x8(qa), as_bf16x8(kreg[kk]), sacc);
      pacc = mfma32(as_bf16x8(da), as_bf16x8(vreg[kk]), pacc);
    }
    // tiles that cross the diagonal or a document end are masked element by element
    const bool need_mask = (a.causal && qt0 < kb0 + kKvBK - 1) || qt0 + kKvBQ > e || kb0 + kKvBK > e;
    float p[16], ds[16];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float4 l4 = *reinterpret_cast<const float4*>(sf + 32 * role + 8 * gq + 4 * half);
      const float4 d4 = *reinterpret_cast<const float4*>(sf + kKvBQ + 32 * role + 8 * gq + 4 * half);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int i = 4 * gq + x;
        p[i] = fast_exp2(fmaf(sacc[i], a.sl2, -lv[x]));
        ds[i] = pacc[i] - dv[x];
      }
    }
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = qb0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (qq >= e || kj >= e || (a.causal && kj > qq)) p[i] = 0.f;
      }
    }
    // P then dS, each as two MFMA steps (accumulator elements 8*mm .. 8*mm+7),
    // published for the partner wave (and read back by this one below)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int b = 8 * mm;
      xch[(w * 4 + mm) * 64 + lane] = make_uint4(pack_bf16x2(p[b], p[b + 1]), pack_bf16x2(p[b + 2], p[b + 3]),
                                                 pack_bf16x2(p[b + 4], p[b + 5]), pack_bf16x2(p[b + 6], p[b + 7]));
      xch[(w * 4 + 2 + mm) * 64 + lane] = make_uint4(pack_bf16x2(p[b] * ds[b], p[b + 1] * ds[b + 1]),
                                                     pack_bf16x2(p[b + 2] * ds[b + 2], p[b + 3] * ds[b + 3]),
                                                     pack_bf16x2(p[b + 4] * ds[b + 4], p[b + 5] * ds[b + 5]),
                                                     pack_bf16x2(p[b + 6] * ds[b + 6], p[b + 7] * ds[b + 7]));
    }
    __syncthreads();  // both blocks' P and dS are visible

    // ---- dV^T += dO^T P and dK^T += Q^T dS over both query blocks, for this
    // wave's half of the columns; A operands by transposing reads of dO and Q
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int owner = kgrp + 4 * qb;  // the wave that computed block qb for these keys
      uint4 opnd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) opnd[j] = xch[(owner * 4 + j) * 64 + lane];
#pragma unroll
      for (int c = 0; c < CBH; ++c) {
        const int c0 = 32 * (role * CBH + c);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          dvacc[c] = mfma32(a_from_rows<D>(dos, 32 * qb + 16 * mm, c0, lane), as_bf16x8(opnd[mm]), dvacc[c]);
          dkacc[c] = mfma32(a_from_rows<D>(qs, 32 * qb + 16 * mm, c0, lane), as_bf16x8(opnd[2 + mm]), dkacc[c]);
        }
      }
    }

    if (more) store(smem_raw + ((t + 1) & 1) * STAGE_BYTES);
    __syncthreads();
  }

  if (kj < e) {
    bf16* ko = a.dk + base + (size_t)kj * rs;
    bf16* vo = a.dv + base + (size_t)kj * rs;
#pragma unroll
    for (int c = 0; c < CBH; ++c)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = 32 * (role * CBH + c) + 8 * gq + 4 * half;
        *reinterpret_cast<uint2*>(ko + col) = pack4_scaled(dkacc[c], 4 * gq, a.scale);
        *reinterpret_cast<uint2*>(vo + col) = pack4_scaled(dvacc[c], 4 * gq, 1.f);
      }
  }
}

}  // namespace

namespace uly_host {

int launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, const AttnGeom& g, void* stream) {
  BwdArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = static_cast<const bf16*>(o);
  a.dout = static_cast<const bf16*>(dout);
  a.lse = lse;
  a.delta = delta;
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
  const int maxlen = g.cu ? g.max_doc_len : g.N;
  hipStream_t st = (hipStream_t)stream;

  const long long rows = (long long)a.units * g.N;
  const int rpb = kThreads / (g.d / 8);
  const long long dblocks = (rows + rpb - 1) / rpb;
  if (dblocks > 0x7fffffffLL) return ULY_ESHAPE;

  BwdArgs aq = a;
  aq.nslots = (maxlen + kDqBQ - 1) / kDqBQ;
  const long long qblocks = (long long)aq.nslots * a.ndoc * a.units;
  BwdArgs akv = a;
  akv.nslots = (maxlen + kKvBK - 1) / kKvBK;
  const long long kvblocks = (long long)akv.nslots * a.ndoc * a.units;
  if (qblocks > 0x7fffffffLL || kvblocks > 0x7fffffffLL) return ULY_ESHAPE;

  if (g.d == 64) {
    hipLaunchKernelGGL(delta_bf16_kernel<64>, dim3((unsigned)dblocks), dim3(kThreads), 0, st, a.o, a.dout,
                       delta, g.N, g.Hl, rows);
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<64>, dim3((unsigned)kvblocks), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL(attn_dq_bf16_kernel<64>, dim3((unsigned)qblocks), dim3(kThreads), 0, st, aq);
  } else {
    hipLaunchKernelGGL(delta_bf16_kernel<128>, dim3((unsigned)dblocks), dim3(kThreads), 0, st, a.o, a.dout,
                       delta, g.N, g.Hl, rows);
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<128>, dim3((unsigned)kvblocks), dim3(kKvThreads), 0, st, akv);
    hipLaunchKernelGGL(attn_dq_bf16_kernel<128>, dim3((unsigned)qblocks), dim3(kThreads), 0, st, aq);
  }
  return launch_status();
}

}  // namespace uly_host

extern "C" size_t ulysses_attn_bwd_workspace_bytes(int sp, int B, int N, int Hl, int d, int dtype) {
  if (sp <= 0 || B <= 0 || N <= 0 || Hl <= 0) return 0;
  if (!uly_host::dtype_ok(dtype) || !uly_host::head_dim_ok(d)) return 0;
  // D = rowsum(dO * O): one float per (rank, batch row, head, token).
  return (size_t)sp * B * Hl * N * sizeof(float);
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
