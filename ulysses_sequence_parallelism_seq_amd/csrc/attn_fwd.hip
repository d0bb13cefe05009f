// Attention forward on gfx950 matrix cores (bf16 inputs, fp32 accumulation),
// and the ulysses_attn_fwd entry point.
//
// What it computes (congresoia365 article, "Cómo Funciona Ulysses": each rank
// runs standard attention over all N tokens of its heads; HF guide,
// "sp_attn_implementation": packed samples stay apart; congresoia365,
// "El Desafío ...": O(N) memory, no N x N matrix): for every (row, head),
// O = softmax(Q K^T / sqrt(d) + mask) V and lse = ln sum exp(...), with the
// mask allowing key j for query i iff both sit in the same document and
// (not causal or j <= i).
//
// Kernel design (one workgroup = 8 waves = a tile of 256 queries of one
// document of one (row, head); the waves share each staged K/V tile):
//   * Each wave owns 32 queries. It computes S^T = K Q^T with the 32x32x16
//     bf16 MFMA: K (A operand) comes from LDS, Q^T (B operand) stays in
//     registers for the whole kernel. In the S^T accumulator layout a lane
//     holds one query and 16 keys, so row max and row sum are in-register
//     except for one exchange between the two half-waves.
//   * Online softmax in the exp2 domain (log2(e)/sqrt(d) folded into the
//     exponent's FMA), with a lazily moved running max (see kSumLimit). P^T is packed to bf16 straight from the accumulator and is
//     the B operand of O^T += V^T P^T, again a 32x32x16 MFMA, whose A
//     operand V^T comes from the row-major V tile through gfx950's
//     transposing LDS reads. The MFMA k index is mapped to keys so that each
//     lane's own P values form its B operand (no data movement between
//     lanes). The O^T accumulator has one query per lane, so the rescale by
//     the running-max correction is a per-lane scalar.
//   * K/V tiles of 64 keys are staged in LDS (row-major, swizzled 16-byte
//     chunks), double-buffered: direct-to-LDS loads of tile t+1 are issued
//     before the math of tile t and waited for before its barrier, one
//     barrier per tile. The two stages are separate arrays addressed by
//     name (the loop is unrolled by two), so the compiler can tell the
//     stage being loaded from the one being read. Loads go through buffer
//     resources ending at the document end (zeros past it; per-lane offsets
//     fixed per kernel).
//   * Documents: a query tile never straddles a document; its keys run from
//     the document start to the tile's last query (causal) or the document
//     end. Only the tiles that cross the diagonal or the document end are
//     masked element by element.
//   * Launch order: query-tile index descending (longest causal work first),
//     then document, then (row, head). Workgroups are dealt round-robin to
//     the 8 XCDs, so with (row, head) fastest each XCD keeps to a few heads
//     and its L2 serves their K/V tiles to all the XCD's workgroups.

#include <math.h>

#include "common.h"
#include "launch.h"

namespace {

using namespace uly;

constexpr int kBQ = 256;  // queries per workgroup (32 per wave)
constexpr int kBK = 64;   // keys per K/V tile
constexpr int kThreads = 512;  // 8 waves sharing each K/V tile

template <int D>
struct FwdSmem {
  using L = RowTile<D>;  // K and V tiles, row-major, swizzled chunks
  static constexpr int TILE = kBK * L::RS;
};

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const int* cu;
  int ndoc;
  int nq_slots;  // query tiles per document slot
  int units;     // G * Hl
  int Hl;
  int N;
  int causal;
  float sl2;  // log2(e) / sqrt(d)
  // ring step only: running normalised O (fp32, same layout as o), the step,
  // and the ring size and batch rows that make up the G = sp * B stacked rows
  float* o_acc;
  int step, sp, B;
  // persistent launch: the tile-queue counters (TileQueue) in the caller's
  // workspace; nullptr: one tile per workgroup
  int* sched;
};

// Lazy rescale: the running max m used in the exponentials only moves when
// a tile's row sum of exp2(x - m) would reach 2^64 (or overflow, as on a
// row's first keys, where m is not set yet). Until then P may exceed 1 by
// that much, which fp32 sums, fp32 accumulators and bf16 MFMA operands hold
// with the same relative precision; the final normalisation uses the same m,
// so the result is the same softmax. Most tiles thus need no row max at all.
constexpr float kSumLimit = 0x1p64f;

// kRing: one step of ring attention. Row g = r * B + b holds rank r's query
// chunk; its keys and values come from chunk j = (r - step) mod sp, the whole
// chunk (j < r, or not causal), its causal diagonal (j == r) or none (j > r).
// The kernel starts from the running state (o_acc, lse) of the previous steps
// and leaves the merged state there; o is written at the rank's last step.
template <int D, bool kRing>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  using S = FwdSmem<D>;
  constexpr int KK = D / 16;  // MFMA k-steps over the head dimension
  constexpr int CB = D / 32;  // 32-wide column blocks of O^T
  // K and V of even tiles, then of odd tiles
  __shared__ __attribute__((aligned(16))) bf16 k0s[S::TILE];
  __shared__ __attribute__((aligned(16))) bf16 v0s[S::TILE];
  __shared__ __attribute__((aligned(16))) bf16 k1s[S::TILE];
  __shared__ __attribute__((aligned(16))) bf16 v1s[S::TILE];

  // ---- which tile
  __shared__ int s_claim[4];
  TileQueue tq;
  tq.init(a.sched, a.nq_slots, a.ndoc, a.units);
  TileId tid_;
  while (tq.next(tid_, s_claim)) {
    const int lvl = tid_.lvl, doc = tid_.doc, unit = tid_.unit;
    const int qslot = a.nq_slots - 1 - lvl;
    int s = 0, e = a.N;
    if (a.cu) {
      s = a.cu[doc];
      e = a.cu[doc + 1];
    }
    const int q0 = s + qslot * kBQ;
    if (q0 >= e) continue;  // the whole workgroup skips the tile

    const int g = unit / a.Hl, hd = unit - (unit / a.Hl) * a.Hl;
    const size_t rs = (size_t)a.Hl * D;
    const size_t base = ((size_t)g * a.N * a.Hl + hd) * D;
    size_t kvbase = base;
    int causal = a.causal;
    bool first = true, last = true;
    if constexpr (kRing) {
      const int r = g / a.B, b = g - (g / a.B) * a.B;
      const int j = r >= a.step ? r - a.step : r - a.step + a.sp;
      if (a.causal && j > r) continue;  // no key of this chunk is visible: the whole workgroup skips the tile
      causal = a.causal && j == r;
      kvbase = ((size_t)(j * a.B + b) * a.N * a.Hl + hd) * D;
      first = a.step == 0;
      last = a.causal ? a.step == r : a.step == a.sp - 1;
    }
    const bf16* qb = a.q + base;
    const bf16* kb = a.k + kvbase;
    const bf16* vb = a.v + kvbase;

    // the lane-derived values are recomputed per tile (the opaque copy keeps
    // them out of the tile loop's live state), the wave index is scalar
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5, l32 = lane & 31;
    const int qi = q0 + 32 * w + l32;  // this lane's query
    FragOffsets<D> fo;
    fo.init(lane);
    const bool qvalid = qi < e;

    // ---- Q^T operand, resident for the whole kernel (rows past the document end read as zero)
    const uint32_t row_bytes = (uint32_t)rs * 2u;
    uint4 qreg[KK];
    {
      const rsrc_t qr = make_rsrc(qb + (size_t)q0 * rs, (long long)(e - q0) * row_bytes);
      const uint32_t qoff = (uint32_t)(32 * w + l32) * row_bytes + (uint32_t)(8 * half) * 2u;
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) qreg[kk] = buf_load16(qr, qoff + 32u * kk);
    }

    const int kend = causal ? min(e, q0 + kBQ) : e;
    const int ntiles = (kend - s + kBK - 1) / kBK;
    // The last key that this wave's queries see: its last query (causal) or
    // the document's last key; none when all 32 queries lie past the
    // document end (a ragged last tile), whose rows are never stored.
    const int wave_klast = q0 + 32 * w >= e ? -1 : causal ? q0 + 32 * w + 31 : e - 1;

    f32x16 oacc[CB];
  #pragma unroll
    for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
      for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
    float m_run = -1e30f, l_run = 0.f;
    if constexpr (kRing) {
      // continue the online softmax from the previous steps: with the running
      // max at lse (log2 units) the earlier keys weigh exactly 1 in total and
      // the normalised O_acc is their weighted sum
      if (!first && qvalid) {
        const float* arow = a.o_acc + base + (size_t)qi * rs;
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const float4 x = *reinterpret_cast<const float4*>(arow + cb * 32 + 8 * gq + 4 * half);
            oacc[cb][4 * gq] = x.x;
            oacc[cb][4 * gq + 1] = x.y;
            oacc[cb][4 * gq + 2] = x.z;
            oacc[cb][4 * gq + 3] = x.w;
          }
        m_run = a.lse[(size_t)unit * a.N + qi] * kLog2e;
        l_run = half == 0 ? 1.f : 0.f;  // the two half-waves' partial sums add up to 1
      }
    }

    TileDma<D, kBK, kThreads / 64> dma;
    dma.init(w, lane, row_bytes);
    auto rsrc_at = [&](const bf16* p, int kt0) {
      return make_rsrc(p + (size_t)kt0 * rs, (long long)(e - kt0) * row_bytes);
    };
    dma.issue(rsrc_at(kb, s), k0s);
    dma.issue(rsrc_at(vb, s), v0s);
    wait_vmem();
    __syncthreads();

    auto step = [&](int t, const bf16* ks, const bf16* vs, const bf16* kn, const bf16* vn) {
      const int kt0 = s + t * kBK;
      if (t + 1 < ntiles) {
        dma.issue(rsrc_at(kb, kt0 + kBK), kn);
        dma.issue(rsrc_at(vb, kt0 + kBK), vn);
      }

      const bool wave_active = kt0 <= wave_klast;
      if (wave_active) {
        // S^T for the tile's 32-key blocks
        constexpr int NB = kBK / 32;
        f32x16 sacc[NB];
  #pragma unroll
        for (int blk = 0; blk < NB; ++blk)
  #pragma unroll
          for (int i = 0; i < 16; ++i) sacc[blk][i] = 0.f;
        // K fragment m (key block m / KK, k-step m % KK) is read PF MFMAs
        // ahead of its use; the scheduling barriers keep that distance
        constexpr int PF = 2;
        auto kfrag = [&](int m) {
          return lds_ld16(ks, fo.row_frag(m / KK, m % KK));
        };
        uint4 kf[PF + 1];
  #pragma unroll
        for (int m = 0; m < PF; ++m) kf[m] = kfrag(m);
  #pragma unroll
        for (int m = 0; m < NB * KK; ++m) {
          if (m + PF < NB * KK) kf[(m + PF) % (PF + 1)] = kfrag(m + PF);
          sacc[m / KK] = mfma32(as_bf16x8(kf[m % (PF + 1)]), as_bf16x8(qreg[m % KK]), sacc[m / KK]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // mask where the tile crosses the diagonal or the document end (scale applied in the exponent)
        const bool need_mask = (causal && kt0 + kBK - 1 > q0) || kt0 + kBK > e;
        if (need_mask) {
  #pragma unroll
          for (int blk = 0; blk < NB; ++blk)
  #pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kt0 + blk * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
              if (key >= e || (causal && key > qi)) sacc[blk][i] = -INFINITY;
            }
        }

        // P^T = exp2(x - m) against the current running max m, optimistically:
        // the tile's row sum shows whether m has fallen too far behind (or, on
        // a row's first keys, was never set). Only then is the tile's row max
        // taken (over both half-waves, which hold different keys of the same
        // query), O and the running sum rescaled and the exponentials redone.
        // The row sum takes the tile's 32 values pairwise before adding them to
        // the running sum: over a long row that adds far fewer roundings than
        // one value at a time (which matters when many terms are alike).
        static_assert(NB == 2, "the pairwise tile sum covers four groups of eight");
        float p[NB][16];
        auto exps = [&]() {
          float ls[2 * NB];
  #pragma unroll
          for (int blk = 0; blk < NB; ++blk)
  #pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
              float* q8 = &p[blk][8 * mm];
  #pragma unroll
              for (int j = 0; j < 8; ++j) q8[j] = fast_exp2(fmaf(sacc[blk][8 * mm + j], a.sl2, -m_run));
              ls[blk * 2 + mm] = ((q8[0] + q8[1]) + (q8[2] + q8[3])) + ((q8[4] + q8[5]) + (q8[6] + q8[7]));
            }
          return (ls[0] + ls[1]) + (ls[2] + ls[3]);
        };
        float lt = exps();
        if (__any(!(lt < kSumLimit))) {
          float mloc = -INFINITY;
  #pragma unroll
          for (int blk = 0; blk < NB; ++blk)
  #pragma unroll
            for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[blk][i]);
          const float m_new = fmaxf(m_run, fmaxf(mloc, swap_halves(mloc)) * a.sl2);
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
  #pragma unroll
          for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
            for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
          lt = exps();
        }
        l_run += lt;
        // packed to bf16 as the B operand of four 16-key MFMA steps
        uint4 pb[2 * NB];
  #pragma unroll
        for (int blk = 0; blk < NB; ++blk)
  #pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const float* q8 = &p[blk][8 * mm];
            pb[blk * 2 + mm] = make_uint4(pack_bf16x2(q8[0], q8[1]), pack_bf16x2(q8[2], q8[3]),
                                          pack_bf16x2(q8[4], q8[5]), pack_bf16x2(q8[6], q8[7]));
          }

        // O^T += V^T P^T: the A operand is V^T read from the row-major V tile
        // with transposing reads; step (blk, mm) covers keys blk*32 + 16*mm ..
        // +15 in the accumulator's row order, which is how P^T sits in pb.
        // V^T fragment m (column block m / (2 NB), step m % (2 NB)) is read PF
        // MFMAs ahead of its use, the distance held by scheduling barriers (left
        // to itself, the scheduler has placed each fragment's reads right before
        // its MFMA, one LDS latency per MFMA)
        constexpr int NV = CB * 2 * NB;
        bf16x8 vf[PF + 1];
  #pragma unroll
        for (int m = 0; m < PF; ++m) vf[m] = a_from_rows_at<D>(vs, fo, m % (2 * NB), m / (2 * NB));
  #pragma unroll
        for (int m = 0; m < NV; ++m) {
          if (m + PF < NV) vf[(m + PF) % (PF + 1)] = a_from_rows_at<D>(vs, fo, (m + PF) % (2 * NB), (m + PF) / (2 * NB));
          oacc[m / (2 * NB)] = mfma32(vf[m % (PF + 1)], as_bf16x8(pb[m % (2 * NB)]), oacc[m / (2 * NB)]);
          __builtin_amdgcn_sched_barrier(0);
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

    // ---- normalise and write O (one query per lane, 4 consecutive columns per store) and lse
    const float l_tot = l_run + swap_halves(l_run);
    if (qvalid) {
      const float inv = 1.f / l_tot;
      if constexpr (kRing) {
        float* arow = a.o_acc + base + (size_t)qi * rs;
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq)
            *reinterpret_cast<float4*>(arow + cb * 32 + 8 * gq + 4 * half) =
                make_float4(oacc[cb][4 * gq] * inv, oacc[cb][4 * gq + 1] * inv, oacc[cb][4 * gq + 2] * inv,
                            oacc[cb][4 * gq + 3] * inv);
      }
      if (last) {
        bf16* orow = a.o + base + (size_t)qi * rs;
  #pragma unroll
        for (int cb = 0; cb < CB; ++cb)
  #pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int c = cb * 32 + 8 * gq + 4 * half;
            *reinterpret_cast<uint2*>(orow + c) = pack4_scaled(oacc[cb], 4 * gq, inv);
          }
      }
      if (half == 0) a.lse[(size_t)unit * a.N + qi] = (m_run + log2f(l_tot)) * kLn2;
    }
    tq.publish(s_claim);  // (its wait for the claim does not wait for the stores)
  }
  tq.finish();
}

// Clears a persistent launch's queue counters (a kernel rather than a memset,
// so that the call can be captured in a graph).
__global__ void sched_clear_kernel(int* p) {
  if (threadIdx.x < kQueueInts) p[threadIdx.x * kCtrStride] = 0;
}

}  // namespace

namespace uly_host {

int launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         const AttnGeom& g, void* stream, int* sched) {
  FwdArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = static_cast<bf16*>(o);
  a.lse = lse;
  a.cu = g.cu;
  a.ndoc = g.ndoc;
  const int maxlen = g.cu ? g.max_doc_len : g.N;
  a.nq_slots = (maxlen + kBQ - 1) / kBQ;
  a.units = g.G * g.Hl;
  a.Hl = g.Hl;
  a.N = g.N;
  a.causal = g.causal;
  a.sl2 = uly::kLog2e / sqrtf((float)g.d);
  a.o_acc = nullptr;
  a.step = 0;
  a.sp = 1;
  a.B = 1;
  a.sched = nullptr;
  const long long blocks = (long long)a.nq_slots * a.ndoc * a.units;
  // the tile decode also forms nq_slots * ndoc * kUnitGroup in int
  const long long span = (long long)a.nq_slots * a.ndoc * (a.units > uly::kUnitGroup ? a.units : uly::kUnitGroup);
  if (span > 0x7fffffffLL) return ULY_ESHAPE;
  hipStream_t st = (hipStream_t)stream;
  long long grid = blocks;
  // Persistent launch when the caller lends the counters: one workgroup per
  // compute unit taking tiles from the per-XCD queues (cleared first).
  const int ncu = sched ? device_cu_count() : 0;
  if (ncu > 0) {
    hipLaunchKernelGGL(sched_clear_kernel, dim3(1), dim3(64), 0, st, sched);
    a.sched = sched;
    grid = blocks < ncu ? blocks : ncu;
  }
  if (g.d == 64)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return launch_status();
}

int launch_ring_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* o_acc, float* lse,
                         const AttnGeom& g, int sp, int B, int step, void* stream, int* sched) {
  FwdArgs a;
  a.q = static_cast<const bf16*>(q);
  a.k = static_cast<const bf16*>(k);
  a.v = static_cast<const bf16*>(v);
  a.o = static_cast<bf16*>(o);
  a.lse = lse;
  a.cu = nullptr;
  a.ndoc = 1;
  a.nq_slots = (g.N + kBQ - 1) / kBQ;
  a.units = g.G * g.Hl;
  a.Hl = g.Hl;
  a.N = g.N;
  a.causal = g.causal;
  a.sl2 = uly::kLog2e / sqrtf((float)g.d);
  a.o_acc = o_acc;
  a.step = step;
  a.sp = sp;
  a.B = B;
  a.sched = nullptr;
  const long long blocks = (long long)a.nq_slots * a.units;
  const long long span = (long long)a.nq_slots * (a.units > uly::kUnitGroup ? a.units : uly::kUnitGroup);
  if (span > 0x7fffffffLL) return ULY_ESHAPE;
  hipStream_t st = (hipStream_t)stream;
  long long grid = blocks;
  // persistent when the caller lends the counters (tiles of ranks this step
  // does not reach are claimed and passed over), else one tile per workgroup
  const int ncu = sched ? device_cu_count() : 0;
  if (ncu > 0) {
    hipLaunchKernelGGL(sched_clear_kernel, dim3(1), dim3(64), 0, st, sched);
    a.sched = sched;
    grid = blocks < ncu ? blocks : ncu;
  }
  if (g.d == 64)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return launch_status();
}

}  // namespace uly_host

namespace {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int* sched,
             const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B, int N, int Hl, int d,
             int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return ULY_EINVAL;
  const int rc = uly_host::check_attn_args(ndoc, max_doc_len, cu_seqlens, sp, B, N, Hl, d, dtype);
  if (rc != ULY_OK) return rc;
  uly_host::AttnGeom g;
  g.G = sp * B;
  g.N = N;
  g.Hl = Hl;
  g.d = d;
  g.cu = cu_seqlens;
  g.ndoc = cu_seqlens ? ndoc : 1;
  g.max_doc_len = cu_seqlens ? max_doc_len : N;
  g.causal = causal ? 1 : 0;
  if (dtype == ULY_F32)
    return uly_host::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                         static_cast<const float*>(v), static_cast<float*>(o), lse, g,
                                         stream);
  return uly_host::launch_attn_fwd_bf16(q, k, v, o, lse, g, stream, sched);
}

}  // namespace

extern "C" int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B,
                                int N, int Hl, int d, int causal, int dtype, void* stream) {
  return attn_fwd(q, k, v, o, lse, nullptr, cu_seqlens, ndoc, max_doc_len, sp, B, N, Hl, d, causal, dtype,
                  stream);
}

extern "C" size_t ulysses_attn_fwd_workspace_bytes(void) { return kQueueBytes; }

extern "C" int ulysses_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                                   void* workspace, size_t workspace_bytes, const int* cu_seqlens, int ndoc,
                                   int max_doc_len, int sp, int B, int N, int Hl, int d, int causal, int dtype,
                                   void* stream) {
  if (!workspace || workspace_bytes < ulysses_attn_fwd_workspace_bytes()) return ULY_EWORKSPACE;
  return attn_fwd(q, k, v, o, lse, static_cast<int*>(workspace), cu_seqlens, ndoc, max_doc_len, sp, B, N, Hl,
                  d, causal, dtype, stream);
}
