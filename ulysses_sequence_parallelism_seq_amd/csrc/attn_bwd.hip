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
//     64-key K/V tiles of its document. Per tile: S^T = K Q^T and
//     dP^T = V dO^T (lane = query, so lse_i and D_i are per-lane scalars),
//     dS^T in registers, then dQ^T += K^T dS^T with K^T staged in LDS.
//   * dkdv kernel, key-stationary: a workgroup owns 128 keys (32 per wave, K
//     and V resident as B operands) and walks 32-query tiles from its first
//     key (causal) to the document end. Per tile: S = Q K^T and dP = dO V^T
//     (lane = key), then dV^T += dO^T P and dK^T += Q^T dS with Q^T and
//     dO^T staged in LDS; the accumulators hold one key per lane, so the
//     final stores are 4 consecutive columns per lane.
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
// A 4-token x 8-column block of a [token][d] tensor, loaded as four 16-byte
// rows; written to LDS row-major and/or transposed ([column][token]).
__device__ __forceinline__ void load_block4(uint4 (&r)[4], const bf16* base, size_t rs, int row0, int c8,
                                            int e) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int row = row0 + x;
    r[x] = row < e ? *reinterpret_cast<const uint4*>(base + (size_t)row * rs + c8 * 8) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_block4_rows(const uint4 (&r)[4], bf16* dst, int stride, int row0,
                                                  int c8) {
#pragma unroll
  for (int x = 0; x < 4; ++x) *reinterpret_cast<uint4*>(dst + (row0 + x) * stride + c8 * 8) = r[x];
}

__device__ __forceinline__ void store_block4_transposed(const uint4 (&r)[4], bf16* dst, int stride,
                                                        int row0, int c8) {
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int wi = c >> 1;
    uint32_t lo, hi;
    if (c & 1) {
      lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
      hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
    } else {
      lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
      hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
    }
    *reinterpret_cast<uint2*>(dst + (c8 * 8 + c) * stride + row0) = make_uint2(lo, hi);
  }
}

// The MFMA A operand of a 16-token step from a transposed LDS row: tokens
// off + 4*half + (0..3) and off + 8 + 4*half + (0..3).
__device__ __forceinline__ bf16x8 a_from_transposed(const bf16* row, int off, int half) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + off + 4 * half);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + off + 8 + 4 * half);
  return as_bf16x8(make_bf16x8_bits(lo, hi));
}

// --------------------------------------------------------------------- dq kernel
constexpr int kDqBQ = 128;  // queries per workgroup
constexpr int kDqBK = 64;   // keys per tile

template <int D>
struct DqSmem {
  static constexpr int KS = D + 8;
  static constexpr int TS = kDqBK + 4;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = kDqBK * KS;
  static constexpr int KT_OFF = 2 * kDqBK * KS;
  static constexpr int ELEMS = 2 * kDqBK * KS + D * TS;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_dq_bf16_kernel(BwdArgs a) {
  using S = DqSmem<D>;
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int BLOCKS = (kDqBK / 4) * (D / 8);  // 4x8 blocks per K (or V) tile
  constexpr int BPT = (BLOCKS + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) bf16 smem[S::ELEMS];

  const int per_level = a.ndoc * a.units;
  const int lvl = blockIdx.x / per_level;
  const int rem = blockIdx.x - lvl * per_level;
  const int doc = rem / a.units;
  const int unit = rem - doc * a.units;
  int s, e;
  doc_range(a, doc, s, e);
  const int q0 = s + (a.nslots - 1 - lvl) * kDqBQ;
  if (q0 >= e) return;

  const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
  const size_t rs = (size_t)a.Hl * D;
  const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int qi = q0 + 32 * w + l32;
  const bool qvalid = qi < e;

  uint4 qreg[KK], doreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const size_t off = base + (size_t)qi * rs + 16 * kk + 8 * half;
    qreg[kk] = qvalid ? *reinterpret_cast<const uint4*>(a.q + off) : make_uint4(0, 0, 0, 0);
    doreg[kk] = qvalid ? *reinterpret_cast<const uint4*>(a.dout + off) : make_uint4(0, 0, 0, 0);
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

  uint4 kr[BPT][4], vr[BPT][4];
  auto load = [&](int kt0) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int id = tid + j * kThreads;
      if (id < BLOCKS) {
        const int kg = id % (kDqBK / 4), cg = id / (kDqBK / 4);
        load_block4(kr[j], a.k + base, rs, kt0 + 4 * kg, cg, e);
        load_block4(vr[j], a.v + base, rs, kt0 + 4 * kg, cg, e);
      }
    }
  };
  load(s);

  for (int t = 0; t < ntiles; ++t) {
    const int kt0 = s + t * kDqBK;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int id = tid + j * kThreads;
      if (id < BLOCKS) {
        const int kg = id % (kDqBK / 4), cg = id / (kDqBK / 4);
        store_block4_rows(kr[j], smem + S::K_OFF, S::KS, 4 * kg, cg);
        store_block4_rows(vr[j], smem + S::V_OFF, S::KS, 4 * kg, cg);
        store_block4_transposed(kr[j], smem + S::KT_OFF, S::TS, 4 * kg, cg);
      }
    }
    __syncthreads();
    if (t + 1 < ntiles) load(kt0 + kDqBK);

    const bool wave_active = !a.causal || kt0 <= q0 + 32 * w + 31;
    if (wave_active) {
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[blk][i] = pacc[blk][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int off = (blk * 32 + l32) * S::KS + 16 * kk + 8 * half;
          const uint4 ka = *reinterpret_cast<const uint4*>(smem + S::K_OFF + off);
          const uint4 va = *reinterpret_cast<const uint4*>(smem + S::V_OFF + off);
          sacc[blk] = mfma32(as_bf16x8(ka), as_bf16x8(qreg[kk]), sacc[blk]);
          pacc[blk] = mfma32(as_bf16x8(va), as_bf16x8(doreg[kk]), pacc[blk]);
        }
      }
      const bool need_mask = (a.causal && kt0 + kDqBK - 1 > q0) || kt0 + kDqBK > e;
      uint4 dsb[4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * mm + j;
            float p = fast_exp2(sacc[blk][i] * a.sl2 - lse2);
            if (need_mask) {
              const int key = kt0 + blk * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
              if (key >= e || (a.causal && key > qi)) p = 0.f;
            }
            ds[j] = p * (pacc[blk][i] - dlt);
          }
          dsb[blk * 2 + mm] = make_uint4(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3]),
                                         pack_bf16x2(ds[4], ds[5]), pack_bf16x2(ds[6], ds[7]));
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16* ktrow = smem + S::KT_OFF + (cb * 32 + l32) * S::TS;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int koff = (st >> 1) * 32 + (st & 1) * 16;
          dqacc[cb] = mfma32(a_from_transposed(ktrow, koff, half), as_bf16x8(dsb[st]), dqacc[cb]);
        }
      }
    }
  }

  if (qvalid) {
    bf16* out = a.dq + base + (size_t)qi * rs;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int c = cb * 32 + 8 * gq + 4 * half;
        *reinterpret_cast<uint2*>(out + c) = pack4_scaled(dqacc[cb], 4 * gq, a.scale);
      }
  }
}

// ------------------------------------------------------------------- dkdv kernel
constexpr int kKvBK = 128;  // keys per workgroup
constexpr int kKvBQ = 32;   // queries per tile

template <int D>
struct KvSmem {
  static constexpr int RS = D + 8;        // row-major Q / dO stride
  static constexpr int TS = kKvBQ + 4;    // transposed Q^T / dO^T stride
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = kKvBQ * RS;
  static constexpr int QT_OFF = 2 * kKvBQ * RS;
  static constexpr int DOT_OFF = QT_OFF + D * TS;
  static constexpr int ELEMS = 2 * kKvBQ * RS + 2 * D * TS;  // bf16 elements
  static constexpr int STAGE_BYTES = ELEMS * 2 + 2 * kKvBQ * 4;  // + lse2 and D
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using S = KvSmem<D>;
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int BLOCKS = (kKvBQ / 4) * (D / 8);  // 4x8 blocks of one Q (or dO) tile
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * S::STAGE_BYTES];

  const int per_level = a.ndoc * a.units;
  const int lvl = blockIdx.x / per_level;
  const int rem = blockIdx.x - lvl * per_level;
  const int doc = rem / a.units;
  const int unit = rem - doc * a.units;
  int s, e;
  doc_range(a, doc, s, e);
  const int kb0 = s + lvl * kKvBK;  // causal: low key blocks have the most queries, so they go first
  if (kb0 >= e) return;

  const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
  const size_t rs = (size_t)a.Hl * D;
  const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int kj = kb0 + 32 * w + l32;
  const bool kvalid = kj < e;

  uint4 kreg[KK], vreg[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const size_t off = base + (size_t)kj * rs + 16 * kk + 8 * half;
    kreg[kk] = kvalid ? *reinterpret_cast<const uint4*>(a.k + off) : make_uint4(0, 0, 0, 0);
    vreg[kk] = kvalid ? *reinterpret_cast<const uint4*>(a.v + off) : make_uint4(0, 0, 0, 0);
  }

  const int qstart = a.causal ? kb0 : s;
  const int ntiles = (e - qstart + kKvBQ - 1) / kKvBQ;
  const float* lse_u = a.lse + (size_t)unit * a.N;
  const float* dl_u = a.delta + (size_t)unit * a.N;

  f32x16 dkacc[CB], dvacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[cb][i] = dvacc[cb][i] = 0.f;

  // staging: threads [0, 128) carry Q blocks, [128, 256) dO blocks; threads
  // [0, 32) also the tile's lse (log2 units), [32, 64) its D.
  const int which = tid >> 7, bid = tid & 127;
  const bool has_block = bid < BLOCKS;
  const int qg = bid % (kKvBQ / 4), cg = bid / (kKvBQ / 4);
  const bf16* src = which ? a.dout + base : a.q + base;
  uint4 r[4];
  float sv = 0.f;
  auto load = [&](int qt0) {
    if (has_block) load_block4(r, src, rs, qt0 + 4 * qg, cg, e);
    if (tid < 64) {
      const int qq = qt0 + (tid & 31);
      if (tid < 32) sv = qq < e ? lse_u[qq] * kLog2e : 0.f;
      else sv = qq < e ? dl_u[qq] : 0.f;
    }
  };
  auto store = [&](uint8_t* stage) {
    bf16* sm = reinterpret_cast<bf16*>(stage);
    float* sf = reinterpret_cast<float*>(stage + S::ELEMS * 2);
    if (has_block) {
      store_block4_rows(r, sm + (which ? S::DO_OFF : S::Q_OFF), S::RS, 4 * qg, cg);
      store_block4_transposed(r, sm + (which ? S::DOT_OFF : S::QT_OFF), S::TS, 4 * qg, cg);
    }
    if (tid < 64) sf[tid] = sv;
  };

  load(qstart);
  store(smem_raw);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int qt0 = qstart + t * kKvBQ;
    const uint8_t* stage = smem_raw + (t & 1) * S::STAGE_BYTES;
    const bf16* sm = reinterpret_cast<const bf16*>(stage);
    const float* sf = reinterpret_cast<const float*>(stage + S::ELEMS * 2);
    const bool more = t + 1 < ntiles;
    if (more) load(qt0 + kKvBQ);

    const bool wave_active = !a.causal || qt0 + kKvBQ - 1 >= kb0 + 32 * w;
    if (wave_active) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = l32 * S::RS + 16 * kk + 8 * half;
        const uint4 qa = *reinterpret_cast<const uint4*>(sm + S::Q_OFF + off);
        const uint4 da = *reinterpret_cast<const uint4*>(sm + S::DO_OFF + off);
        sacc = mfma32(as_bf16x8(qa), as_bf16x8(kreg[kk]), sacc);
        pacc = mfma32(as_bf16x8(da), as_bf16x8(vreg[kk]), pacc);
      }
      // lane = key kj; element i is query qt0 + 8*(i/4) + 4*half + (i%4)
      const bool need_mask = (a.causal && qt0 < kb0 + kKvBK - 1) || qt0 + kKvBQ > e || kb0 + kKvBK > e;
      uint4 pb[2], dsb[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 l4 = *reinterpret_cast<const float4*>(sf + 8 * gq + 4 * half);
        const float4 d4 = *reinterpret_cast<const float4*>(sf + kKvBQ + 8 * gq + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        float p[4], ds[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 4 * gq + x;
          p[x] = fast_exp2(sacc[i] * a.sl2 - lv[x]);
          if (need_mask) {
            const int qq = qt0 + 8 * gq + 4 * half + x;
            if (qq >= e || !kvalid || (a.causal && kj > qq)) p[x] = 0.f;
          }
          ds[x] = p[x] * (pacc[i] - dv[x]);
        }
        // step mm = gq / 2 holds accumulator elements 8*mm .. 8*mm+7
        const int mm = gq >> 1;
        if ((gq & 1) == 0) {
          pb[mm].x = pack_bf16x2(p[0], p[1]);
          pb[mm].y = pack_bf16x2(p[2], p[3]);
          dsb[mm].x = pack_bf16x2(ds[0], ds[1]);
          dsb[mm].y = pack_bf16x2(ds[2], ds[3]);
        } else {
          pb[mm].z = pack_bf16x2(p[0], p[1]);
          pb[mm].w = pack_bf16x2(p[2], p[3]);
          dsb[mm].z = pack_bf16x2(ds[0], ds[1]);
          dsb[mm].w = pack_bf16x2(ds[2], ds[3]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const bf16* dotrow = sm + S::DOT_OFF + (cb * 32 + l32) * S::TS;
        const bf16* qtrow = sm + S::QT_OFF + (cb * 32 + l32) * S::TS;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          dvacc[cb] = mfma32(a_from_transposed(dotrow, 16 * mm, half), as_bf16x8(pb[mm]), dvacc[cb]);
          dkacc[cb] = mfma32(a_from_transposed(qtrow, 16 * mm, half), as_bf16x8(dsb[mm]), dkacc[cb]);
        }
      }
    }
    if (more) store(smem_raw + ((t + 1) & 1) * S::STAGE_BYTES);
    __syncthreads();
  }

  if (kvalid) {
    bf16* ko = a.dk + base + (size_t)kj * rs;
    bf16* vo = a.dv + base + (size_t)kj * rs;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int c = cb * 32 + 8 * gq + 4 * half;
        *reinterpret_cast<uint2*>(ko + c) = pack4_scaled(dkacc[cb], 4 * gq, a.scale);
        *reinterpret_cast<uint2*>(vo + c) = pack4_scaled(dvacc[cb], 4 * gq, 1.f);
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
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<64>, dim3((unsigned)kvblocks), dim3(kThreads), 0, st, akv);
    hipLaunchKernelGGL(attn_dq_bf16_kernel<64>, dim3((unsigned)qblocks), dim3(kThreads), 0, st, aq);
  } else {
    hipLaunchKernelGGL(delta_bf16_kernel<128>, dim3((unsigned)dblocks), dim3(kThreads), 0, st, a.o, a.dout,
                       delta, g.N, g.Hl, rows);
    hipLaunchKernelGGL(attn_dkdv_bf16_kernel<128>, dim3((unsigned)kvblocks), dim3(kThreads), 0, st, akv);
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
