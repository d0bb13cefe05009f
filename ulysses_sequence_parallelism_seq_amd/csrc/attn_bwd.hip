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
// off0 is the block's byte offset from the tile start; rows past the
// resource's range (the document end) read as zero.
__device__ __forceinline__ void load_block4(uint4 (&r)[4], rsrc_t rsrc, uint32_t off0, uint32_t row_bytes) {
#pragma unroll
  for (int x = 0; x < 4; ++x) r[x] = buf_load16(rsrc, off0 + x * row_bytes);
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
    const uint32_t lo = (c & 1) ? pack_hi16(w0[wi], w1[wi]) : pack_lo16(w0[wi], w1[wi]);
    const uint32_t hi = (c & 1) ? pack_hi16(w2[wi], w3[wi]) : pack_lo16(w2[wi], w3[wi]);
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

  const uint32_t row_bytes = (uint32_t)rs * 2u;
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

  static_assert(BPT == 1, "one 4x8 block of K and of V per thread");
  uint4 kr[BPT][4], vr[BPT][4];
  // this thread's block: keys 4*(tid % 16) .. +3, columns 8*(tid / 16) .. +7
  const uint32_t blk_off = (uint32_t)(4 * (tid % (kDqBK / 4))) * row_bytes + (uint32_t)(tid / (kDqBK / 4)) * 16u;
  auto load = [&](int kt0) {
    if (tid < BLOCKS) {
      const long long span = (long long)(e - kt0) * row_bytes;
      load_block4(kr[0], make_rsrc(a.k + base + (size_t)kt0 * rs, span), blk_off, row_bytes);
      load_block4(vr[0], make_rsrc(a.v + base + (size_t)kt0 * rs, span), blk_off, row_bytes);
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
      if (need_mask) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt0 + blk * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key >= e || (a.causal && key > qi)) sacc[blk][i] = -INFINITY;
          }
      }
      uint4 dsb[4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * mm + j;
            const float p = fast_exp2(fmaf(sacc[blk][i], a.sl2, -lse2));
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
constexpr int kKvBK = 128;  // keys per workgroup (32 per wave)
constexpr int kKvBQ = 64;   // queries per tile (two 32-query MFMA blocks)

template <int D>
struct KvSmem {
  static constexpr int RS = D + 8;        // row-major Q / dO stride (bf16)
  static constexpr int TS = kKvBQ + 4;    // transposed Q^T / dO^T stride (bf16)
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = kKvBQ * RS;
  static constexpr int QT_OFF = 2 * kKvBQ * RS;
  static constexpr int DOT_OFF = QT_OFF + D * TS;
  static constexpr int ELEMS = 2 * kKvBQ * RS + 2 * D * TS;      // bf16 elements
  static constexpr int STAGE_BYTES = ELEMS * 2 + 2 * kKvBQ * 4;  // + lse (log2 units) and D
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_dkdv_bf16_kernel(BwdArgs a) {
  using S = KvSmem<D>;
  constexpr int KK = D / 16, CB = D / 32;
  constexpr int BLOCKS = (kKvBQ / 4) * (D / 8);  // 4x8 blocks of one Q (or dO) tile
  constexpr int BPT = (BLOCKS + kThreads - 1) / kThreads;
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
  const int wk0 = kb0 + 32 * w;  // first key of this wave

  const uint32_t row_bytes = (uint32_t)rs * 2u;
  uint4 kreg[KK], vreg[KK];
  {
    const long long span = (long long)(e - kb0) * row_bytes;
    const rsrc_t kr = make_rsrc(a.k + base + (size_t)kb0 * rs, span);
    const rsrc_t vr = make_rsrc(a.v + base + (size_t)kb0 * rs, span);
    const uint32_t off = (uint32_t)(32 * w + l32) * row_bytes + (uint32_t)(8 * half) * 2u;
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

  f32x16 dkacc[CB], dvacc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkacc[cb][i] = dvacc[cb][i] = 0.f;

  // staging: every thread carries one 4x8 block of Q and the same block of dO
  // (BPT per thread); threads [0, 64) also the tile's lse (log2 units), [64, 128) its D.
  uint4 rq[BPT][4], rd[BPT][4];
  float sv = 0.f;
  auto load = [&](int qt0) {
    const long long span = (long long)(e - qt0) * row_bytes;
    const rsrc_t qr = make_rsrc(a.q + base + (size_t)qt0 * rs, span);
    const rsrc_t dr = make_rsrc(a.dout + base + (size_t)qt0 * rs, span);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int id = tid + j * kThreads;
      if (id < BLOCKS) {
        const int qg = id % (kKvBQ / 4), cg = id / (kKvBQ / 4);
        const uint32_t off0 = (uint32_t)(4 * qg) * row_bytes + (uint32_t)cg * 16u;
        load_block4(rq[j], qr, off0, row_bytes);
        load_block4(rd[j], dr, off0, row_bytes);
      }
    }
    if (tid < 2 * kKvBQ) {
      const int qq = qt0 + (tid % kKvBQ);
      if (tid < kKvBQ) sv = qq < e ? lse_u[qq] * kLog2e : 0.f;
      else sv = qq < e ? dl_u[qq] : 0.f;
    }
  };
  auto store = [&](uint8_t* stage) {
    bf16* sm = reinterpret_cast<bf16*>(stage);
    float* sf = reinterpret_cast<float*>(stage + S::ELEMS * 2);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int id = tid + j * kThreads;
      if (id < BLOCKS) {
        const int qg = id % (kKvBQ / 4), cg = id / (kKvBQ / 4);
        store_block4_rows(rq[j], sm + S::Q_OFF, S::RS, 4 * qg, cg);
        store_block4_transposed(rq[j], sm + S::QT_OFF, S::TS, 4 * qg, cg);
        store_block4_rows(rd[j], sm + S::DO_OFF, S::RS, 4 * qg, cg);
        store_block4_transposed(rd[j], sm + S::DOT_OFF, S::TS, 4 * qg, cg);
      }
    }
    if (tid < 2 * kKvBQ) sf[tid] = sv;
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

    const bool need_mask = (a.causal && qt0 < kb0 + kKvBK - 1) || qt0 + kKvBQ > e || kb0 + kKvBK > e;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = qt0 + 32 * qb;
      // causal: a 32-query block that ends before this wave's first key adds nothing
      if (a.causal && qb0 + 31 < wk0) continue;
      f32x16 sacc, pacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int off = (32 * qb + l32) * S::RS + 16 * kk + 8 * half;
        const uint4 qa = *reinterpret_cast<const uint4*>(sm + S::Q_OFF + off);
        const uint4 da = *reinterpret_cast<const uint4*>(sm + S::DO_OFF + off);
        sacc = mfma32(as_bf16x8(qa), as_bf16x8(kreg[kk]), sacc);
        pacc = mfma32(as_bf16x8(da), as_bf16x8(vreg[kk]), pacc);
      }
      // lane = key kj; element i is query qb0 + 8*(i/4) + 4*half + (i%4)
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = qb0 + 8 * (i >> 2) + 4 * half + (i & 3);
          if (qq >= e || !kvalid || (a.causal && kj > qq)) sacc[i] = -INFINITY;
        }
      }
      uint4 pb[2], dsb[2];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 l4 = *reinterpret_cast<const float4*>(sf + 32 * qb + 8 * gq + 4 * half);
        const float4 d4 = *reinterpret_cast<const float4*>(sf + kKvBQ + 32 * qb + 8 * gq + 4 * half);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        float p[4], ds[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          p[x] = fast_exp2(fmaf(sacc[4 * gq + x], a.sl2, -lv[x]));
          ds[x] = p[x] * (pacc[4 * gq + x] - dv[x]);
        }
        // MFMA step mm = gq / 2 takes accumulator elements 8*mm .. 8*mm+7
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
        const bf16* dotrow = sm + S::DOT_OFF + (cb * 32 + l32) * S::TS + 32 * qb;
        const bf16* qtrow = sm + S::QT_OFF + (cb * 32 + l32) * S::TS + 32 * qb;
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
