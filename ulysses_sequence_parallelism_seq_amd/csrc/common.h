// Shared helpers of the gfx950 kernels: vector types, MFMA wrappers, host-side
// argument checks and launch error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ulysses.h"

namespace uly {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l (h = l / 32) supplies
// A[m = l % 32][k = 8h .. 8h+7] and B[k = 8h .. 8h+7][n = l % 32]; the result
// element acc[i] of lane l is C[m = 8(i/4) + 4h + (i%4)][n = l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint4 make_bf16x8_bits(uint2 lo, uint2 hi) {
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float float2_t;

// Round-to-nearest-even fp32 -> bf16 of two values, packed low|high (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zero without touching memory (raw buffer, stride 0, range-checked
// on the per-lane offset). Used to zero-fill rows past a document end.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// Direct global -> LDS load (buffer_load_dwordx4 ... lds): lane i's 16 bytes
// from byte offset voff land at byte 16*i of the wave's 1 KB LDS window that
// starts at lds (wave-uniform); offsets past the resource range write zeros
// (both checked on gfx950). Completion is waited for with wait_vmem(). The
// compiler makes LDS reads wait for such loads unless it can tell the two
// apart, so the stages they fill are separate __shared__ arrays, each
// addressed by name.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, const void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)const_cast<void*>(lds), 16, (int)voff, 0, 0, 0);
}
// Same with 4 bytes per lane (lane i lands at byte 4*i of a 256-byte window).
__device__ __forceinline__ void buf_load4_lds(rsrc_t r, const void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)const_cast<void*>(lds), 4, (int)voff, 0, 0, 0);
}
// s_waitcnt vmcnt(0), leaving the other counters alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0) alone (vmcnt 63, expcnt 7), then s_barrier: a workgroup
// barrier that orders LDS accesses but lets global loads stay in flight.
__device__ __forceinline__ void barrier_lds_only() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-bit halves of two words: (hi.lo16 << 16 | lo.lo16) and (hi.hi16 << 16 | lo.hi16).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t lo, uint32_t hi) {
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Elements i0 .. i0+3 of an accumulator, times s, as four packed bf16.
__device__ __forceinline__ uint2 pack4_scaled(const f32x16& v, int i0, float s) {
  return make_uint2(pack_bf16x2(v[i0] * s, v[i0 + 1] * s), pack_bf16x2(v[i0 + 2] * s, v[i0 + 3] * s));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunks addressed by lanes
// 4m + i/4 of its group, for m = 0..3 (layout checked on gfx950).
__device__ __forceinline__ uint2 lds_read_tr16(const bf16* p) {
  const lds_v4i16* a = (const lds_v4i16*)(const __attribute__((address_space(3))) void*)(p);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4i16*>(a)));
}

// Layout of a [token][d] bf16 tile in LDS: unpadded rows of 2d bytes whose
// 16-byte chunk c sits at chunk c ^ swz(r) (for d = 64 the low 3 bits of
// swz). swz makes three access patterns free of bank conflicts (with 32 or
// 64 banks): 16-byte reads of one chunk from 16 consecutive rows (MFMA
// operands), the transposing reads of a_from_rows (4 rows x 4 half-chunks
// per 16 lanes) and 16-byte stores of whole rows (staging). Unpadded rows
// also let a wave's direct-to-LDS load fill whole rows.
__host__ __device__ constexpr int swz(int r) { return ((10 * (r & 3)) & 15) ^ ((r >> 2) & 3); }

// swz permutes the 16 chunks of a 256-byte row (a chunk never leaves its row).
constexpr bool swz_stays_in_row() {
  for (int r = 0; r < 16; ++r)
    for (int c = 0; c < 16; ++c)
      if ((c ^ swz(r)) < 0 || (c ^ swz(r)) > 15) return false;
  return true;
}
static_assert(swz_stays_in_row(), "swizzled chunk index must stay within the row");

template <int D>
struct RowTile {
  static constexpr int RS = D;           // row stride (bf16 elements)
  static constexpr int CHUNKS = D / 8;   // 16-byte chunks per row
  __host__ __device__ static __forceinline__ int chunk_key(int row) { return swz(row) & (CHUNKS - 1); }
  // element offset of (row, col); col is a multiple of 4
  __host__ __device__ static __forceinline__ int off(int row, int col) {
    return row * RS + ((((col >> 3) ^ chunk_key(row)) << 3) | (col & 7));
  }
};

// Global -> LDS staging of a kRows-token tile of one [token][d] tensor with
// direct-to-LDS loads, by kWaves waves: wave w fills rows
// [w * kRows / kWaves, (w + 1) * kRows / kWaves), 1 KB (64 / (D/8) whole rows)
// per instruction. Lane i lands on physical chunk i % (D/8) of its row, so it
// fetches the logical chunk that the RowTile swizzle keeps there. The buffer
// range ends at the document end: rows past it are written as zeros.
template <int D, int kRows, int kWaves>
struct TileDma {
  static constexpr int CHUNKS = D / 8;
  static constexpr int ROWS_PER_OP = 64 / CHUNKS;
  static constexpr int ROWS_PER_WAVE = kRows / kWaves;
  static constexpr int OPS = ROWS_PER_WAVE / ROWS_PER_OP;
  static_assert(OPS >= 1 && OPS * ROWS_PER_OP == ROWS_PER_WAVE, "a wave fills whole 1 KB windows");
  uint32_t voff[OPS];
  int lds_off[OPS];

  __device__ __forceinline__ void init(int w, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int j = 0; j < OPS; ++j) {
      const int row0 = ROWS_PER_WAVE * w + ROWS_PER_OP * j;
      const int r = row0 + lane / CHUNKS;
      const int c = (lane % CHUNKS) ^ RowTile<D>::chunk_key(r);
      voff[j] = (uint32_t)r * row_bytes + (uint32_t)c * 16u;
      lds_off[j] = row0 * D;
    }
  }
  __device__ __forceinline__ void issue(rsrc_t rs, const bf16* tile) const {
#pragma unroll
    for (int j = 0; j < OPS; ++j) buf_load16_lds(rs, tile + lds_off[j], voff[j]);
  }
};

// Per-lane LDS byte offsets of the two fragment reads made from RowTile<D>
// tiles, in a form that costs one register per pattern. Swizzle keys repeat
// every 16 rows, and a chunk index x + y with x, y on disjoint bits, XORed with
// a key, equals (y ^ key) ^ x; a row is 2D bytes with the chunk in bits 4 and
// up, so each fragment's offset is a lane base XOR a constant, plus a constant
// number of whole rows:
//   * row operand (lane l: row 32 rb + l % 32, columns 16 kk + 8 h .. + 7),
//     the operand RowTile::off reads for MFMAs with k along d:
//     row_frag(rb, kk) = (row ^ (kk << 5)) + rb * 64 D;
//   * the two transposing reads of a_from_rows_at (t0 = 16 j, c0 = 32 cb),
//     whose lane l reads row t0 + 4 (l / 32) + (l % 16) / 4 (+ 8 for the
//     second) at column c0 + 16 ((l / 16) % 2) + 4 (l % 4):
//     (tr_lo or tr_hi) ^ (cb << 6), plus 32 D j.
// Compilers keep offsets they cannot relate as separate registers; with these
// the per-fragment offsets are a few XORs of three registers.
template <int D>
struct FragOffsets {
  uint32_t row, tr_lo, tr_hi;
  __host__ __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5, l32 = lane & 31, p = lane & 15;
    row = (uint32_t)(l32 * 2 * D) + ((uint32_t)(half ^ RowTile<D>::chunk_key(l32)) << 4);
    const int r0 = 4 * half + (p >> 2);  // transposing reads: row of the low half
    const int cl = 2 * ((lane >> 4) & 1) + ((p & 3) >> 1);
    const uint32_t low = (uint32_t)(4 * (p & 1)) * 2u;  // bytes within the chunk
    tr_lo = (uint32_t)(r0 * 2 * D) + ((uint32_t)(cl ^ RowTile<D>::chunk_key(r0)) << 4) + low;
    tr_hi = (uint32_t)((r0 + 8) * 2 * D) + ((uint32_t)(cl ^ RowTile<D>::chunk_key(r0 + 8)) << 4) + low;
  }
  __host__ __device__ __forceinline__ uint32_t row_frag(int rb, int kk) const {
    return (row ^ ((uint32_t)kk << 5)) + (uint32_t)(rb * 64 * D);
  }
};

__device__ __forceinline__ uint4 lds_ld16(const void* tile, uint32_t byte_off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(tile) + byte_off);
}

// MFMA A operand (rows = 32 columns c0 .. c0+31 of a [token][d] LDS tile in
// the RowTile layout; k = 16 tokens from t0), t0 = 16 j and c0 = 32 cb, read
// with two transposing reads at the offsets of FragOffsets. Lane l
// (h = l / 32) receives column c0 + l % 32 of tokens t0 + 4h + (0..3) and
// t0 + 8 + 4h + (0..3): MFMA k index 8h + i is token t0 + 4h + i (i < 4) or
// t0 + 8 + 4h + (i - 4), the same token order as an accumulator's rows.
template <int D>
__device__ __forceinline__ bf16x8 a_from_rows_at(const bf16* tile, const FragOffsets<D>& fo, int j, int cb) {
  const char* t = reinterpret_cast<const char*>(tile) + j * 32 * D;
  const uint32_t x = (uint32_t)cb << 6;
  const uint2 lo = lds_read_tr16(reinterpret_cast<const bf16*>(t + (fo.tr_lo ^ x)));
  const uint2 hi = lds_read_tr16(reinterpret_cast<const bf16*>(t + (fo.tr_hi ^ x)));
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// The same transposing reads addressed for the natural k order: lane l
// (h = l / 32) receives column c0 + l % 32 of rows t0 + 8h + (0..3) (first
// read) and t0 + 8h + 4 + (0..3) (second), so MFMA k index 8h + i is row
// t0 + 8h + i, the order a 16-byte read of a K-contiguous operand gives.
// GEMMs that pair such an operand with a K-strided one read both in this order.
template <int D>
struct NatTrOffsets {
  uint32_t lo, hi;
  __host__ __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5, p = lane & 15;
    const int r0 = 8 * half + (p >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((p & 3) >> 1);
    const uint32_t low = (uint32_t)(4 * (p & 1)) * 2u;
    lo = (uint32_t)(r0 * 2 * D) + ((uint32_t)(cl ^ RowTile<D>::chunk_key(r0)) << 4) + low;
    hi = (uint32_t)((r0 + 4) * 2 * D) + ((uint32_t)(cl ^ RowTile<D>::chunk_key(r0 + 4)) << 4) + low;
  }
};

// MFMA operand (rows = columns c0 .. c0+31 of a [k][D] RowTile<D> LDS tile,
// k = rows t0 .. t0+15 in the natural order), t0 = 16 j, c0 = 32 cb.
template <int D>
__device__ __forceinline__ bf16x8 a_from_rows_nat(const bf16* tile, const NatTrOffsets<D>& no, int j, int cb) {
  const char* t = reinterpret_cast<const char*>(tile) + j * 32 * D;
  const uint32_t x = (uint32_t)cb << 6;
  const uint2 lo = lds_read_tr16(reinterpret_cast<const bf16*>(t + (no.lo ^ x)));
  const uint2 hi = lds_read_tr16(reinterpret_cast<const bf16*>(t + (no.hi ^ x)));
  return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Value held by lane (l ^ 32) of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// Workgroup order: heads (units) in groups of kUnitGroup, each group's tiles
// ordered by level (slowest), then document, then unit (fastest). Consecutive
// workgroups go to consecutive XCDs, so with eight units per group each XCD
// works on one head at a time and its L2 serves every workgroup of that head.
constexpr int kUnitGroup = 8;
struct TileId {
  int lvl, doc, unit;
};
__device__ __forceinline__ TileId decode_tile(int bid, int nslots, int ndoc, int units) {
  const int per_group = nslots * ndoc * kUnitGroup;
  const int gi = bid / per_group;
  const int r = bid - gi * per_group;
  const int ug = min(kUnitGroup, units - gi * kUnitGroup);
  const int per_level = ndoc * ug;
  TileId t;
  t.lvl = r / per_level;
  const int rem = r - t.lvl * per_level;
  t.doc = rem / ug;
  t.unit = gi * kUnitGroup + (rem - t.doc * ug);
  return t;
}

// Tiles of a persistent launch (one workgroup per CU, each taking tile after
// tile until none is left), claimed from eight lists, one per XCD: list x
// holds the tiles of units u = x (mod 8), in four level groups (the longest
// causal work first: levels are ordered by decreasing work), each group unit
// by unit, each unit's part document by document, each document's levels in
// order. Within a group the XCD keeps to one unit (head) and one of its
// documents at a time, so its L2 serves that document's tiles to all its
// workgroups (a unit's documents interleaved level by level cost the
// million-token workload's backward 2.8%); across groups every unit's longest
// tiles come before any unit's shortest ones, so the list ends with short
// tiles even when an XCD has few tiles per workgroup. A workgroup takes from
// its own XCD's list while it lasts, then from the others' lists: XCDs that
// run at a higher clock take over the work of slower ones instead of idling.
// A workgroup's first tile is the one its index names (workgroup b: tile
// b / 8 of list b mod 8, the list of the XCD the hardware deals it to); later
// tiles are claimed with atomic adds on counters in caller memory, one
// 128-byte line per counter (the 256 claims at the end of the first tiles
// would otherwise queue on one line); the forward and dQ kernels send the
// next claim before the current tile's results are written (prefetch,
// publish). Each tile is still computed whole by
// one workgroup, so the results do not depend on the assignment. The last
// workgroup to finish sets the counters back to zero for the next launch on
// the same memory.
// With ctr == nullptr a workgroup handles the one tile blockIdx.x names.
constexpr int kQueueInts = 9;   // 8 claim counters, then the count of finished workgroups
constexpr int kCtrStride = 32;  // ints from one counter to the next
constexpr int kQueueBytes = kQueueInts * kCtrStride * 4;
constexpr int kLevelGroups = 4;

// Tiles in the list of XCD x (the units u = x mod 8 of `units`).
__host__ __device__ __forceinline__ int queue_list_len(int x, int units, int nslots, int ndoc) {
  const int nu = units / kUnitGroup + (x < units % kUnitGroup ? 1 : 0);
  return nu * nslots * ndoc;
}
// Tile i of the list of XCD x: kLevelGroups groups of lg levels (the last one
// holds the nslots % lg left over), each group unit by unit, each unit's part
// document by document, then level by level. Needs i < queue_list_len(...).
__host__ __device__ __forceinline__ TileId queue_decode(int x, int i, int units, int nslots, int ndoc) {
  const int nu = units / kUnitGroup + (x < units % kUnitGroup ? 1 : 0);
  const int lg = (nslots + kLevelGroups - 1) / kLevelGroups;
  const int full = nslots / lg;      // groups of lg levels
  const int gsize = nu * lg * ndoc;  // tiles of one such group
  int grp = i / gsize, nl = lg;
  if (grp >= full) {                 // the last, shorter group
    grp = full;
    nl = nslots - full * lg;
  }
  const int r = i - grp * gsize;     // within the group: unit, then document and level
  const int ui = r / (nl * ndoc), rr = r - ui * (nl * ndoc);
  TileId t;
  t.doc = rr / nl;
  t.lvl = grp * lg + (rr - t.doc * nl);
  t.unit = ui * kUnitGroup + x;
  return t;
}

typedef __attribute__((address_space(1))) int global_int;
// Tiles of a list of n handed out by workgroup index in a grid of `grid`
// workgroups: workgroup b takes tile b / 8 of list b mod 8, so list x gets one
// per workgroup b = x (mod 8) while it lasts; its counter hands out the rest.
__host__ __device__ __forceinline__ int queue_static_count(int x, int grid, int n) {
  return min((grid - x + 7) >> 3, n);
}

struct TileQueue {
  int* ctr;
  int nslots, ndoc, units;
  int x0;         // this workgroup's XCD
  unsigned live;  // lists not yet found exhausted (thread 0)
  int pre;        // thread 0: counter value claimed ahead from list x0
  bool has_pre;   // thread 0: pre holds a claim not yet used
  bool ready;     // thread 0: the coming next() call's tile is already in s_claim
  int calls;      // next() calls so far: the first hands out the tile named by
                  // blockIdx.x (both modes); the parity picks the s_claim pair

  __device__ __forceinline__ void init(int* c, int nslots_, int ndoc_, int units_) {
    ctr = c;
    nslots = nslots_;
    ndoc = ndoc_;
    units = units_;
    x0 = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 7;  // HW_REG_XCC_ID
    live = 0xffu;
    pre = 0;
    has_pre = false;
    ready = false;
    calls = 0;
  }
  __device__ __forceinline__ int list_len(int x) const { return queue_list_len(x, units, nslots, ndoc); }
  __device__ __forceinline__ int static_count(int x) const {
    return queue_static_count(x, (int)gridDim.x, list_len(x));
  }
  // Thread 0: one atomic claim on list x's counter; the tile index is the
  // value plus static_count(x) (the list's length when the workgroup indices
  // already cover the list: no atomic then).
  __device__ __forceinline__ int claim_raw(int x) const {
    if (static_count(x) >= list_len(x)) return list_len(x);
    // The address goes through a vector register: with a uniform one the
    // compiler combines the lanes' adds and broadcasts the result at once,
    // which waits for the atomic right where it is issued.
    global_int* p = (global_int*)(ctr + x * kCtrStride);
    asm volatile("" : "+v"(p));
    return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Thread 0: the next tile (own list first, then the others') into the
  // s_claim pair of next() call c.
  __device__ __forceinline__ void resolve(int* s_claim, int c) {
    int cx = -1, ct = 0;
    for (int k = 0; k < kUnitGroup && cx < 0; ++k) {
      const int x = (x0 + k) & 7;
      if (!((live >> x) & 1u)) continue;
      const int i = ((k == 0 && has_pre) ? pre : claim_raw(x)) + static_count(x);
      if (k == 0) has_pre = false;
      if (i < list_len(x)) {
        cx = x;
        ct = i;
      } else {
        live &= ~(1u << x);
      }
    }
    s_claim[2 * (c & 1)] = cx;
    s_claim[2 * (c & 1) + 1] = ct;
  }
  // The claim of the next tile, in two steps that let its latency pass
  // behind the current tile's work: prefetch() sends the atomic add on the
  // workgroup's own list (early in the tile's last step), publish() puts the
  // next tile into shared memory (once the tile's math is done, before its
  // results are stored, so that the wait for the add's return does not also
  // wait for those stores). Both are for every thread to call; only thread 0
  // acts, and only in the persistent mode.
  __device__ __forceinline__ void prefetch() {
    if (ctr && threadIdx.x == 0 && !has_pre && !ready && ((live >> x0) & 1u)) {
      pre = claim_raw(x0);
      has_pre = true;
    }
  }
  __device__ __forceinline__ void publish(int* s_claim) {
    if (ctr && threadIdx.x == 0 && !ready) {
      resolve(s_claim, calls);
      ready = true;
    }
  }
  // The next tile of this workgroup; false when there is none. Workgroup-
  // uniform; in the persistent mode every thread calls it and every call after
  // the first has one barrier. s_claim: four ints of shared memory, used in
  // two pairs by turns, so that a pair is rewritten only after every wave has
  // passed the barrier that follows its reading.
  __device__ __forceinline__ bool next(TileId& t, int* s_claim) {
    const int c = calls++;
    if (c == 0) {
      const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
      if (!ctr) {
        t = decode_tile(blockIdx.x, nslots, ndoc, units);
        return true;
      }
      if (i < list_len(x)) {
        t = queue_decode(x, i, units, nslots, ndoc);
        return true;
      }
    }
    if (!ctr) return false;
    if (threadIdx.x == 0) {
      if (!ready) resolve(s_claim, c);
      ready = false;
    }
    barrier_lds_only();
    // the same in every lane: saying so keeps the tile's coordinates, and all
    // the addresses and buffer descriptors derived from them, scalar
    const int x = __builtin_amdgcn_readfirstlane(s_claim[2 * (c & 1)]);
    const int i = __builtin_amdgcn_readfirstlane(s_claim[2 * (c & 1) + 1]);
    if (x < 0) return false;
    t = queue_decode(x, i, units, nslots, ndoc);
    return true;
  }
  // After the last next(): counts this workgroup out; the last one resets the counters.
  __device__ __forceinline__ void finish() {
    if (!ctr || threadIdx.x != 0) return;
    if (__hip_atomic_fetch_add(&ctr[8 * kCtrStride], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
        (int)gridDim.x - 1) {
      for (int x = 0; x < kQueueInts; ++x)
        __hip_atomic_store(&ctr[x * kCtrStride], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};
}  // namespace uly

// ---------------------------------------------------------------- host side

namespace uly_host {

inline bool dtype_ok(int dtype) { return dtype == ULY_F32 || dtype == ULY_BF16; }
inline bool head_dim_ok(int d) { return d == 64 || d == 128; }
inline size_t elem_size(int dtype) { return dtype == ULY_F32 ? 4 : 2; }

// Compute units of the current device (the grid of a persistent launch), or 0.
int device_cu_count();

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? ULY_OK : ULY_EHIP;
}

// Checks shared by the attention calls.
inline int check_attn_args(int ndoc, int max_doc_len, const int* cu, int sp, int B, int N, int Hl,
                           int d, int dtype) {
  if (sp <= 0 || B <= 0 || N <= 0 || Hl <= 0 || d <= 0) return ULY_EINVAL;
  if (!dtype_ok(dtype) || !head_dim_ok(d)) return ULY_EUNSUPPORTED;
  if (cu) {
    if (ndoc < 1 || max_doc_len < 1) return ULY_EINVAL;
    if (max_doc_len > N) return ULY_ESHAPE;
  }
  // Token and element offsets are formed in 64 bits; launch sizes in 32;
  // one (row, head) sequence must span < 2 GiB (32-bit buffer offsets).
  if ((long long)sp * B * Hl > (1LL << 24)) return ULY_ESHAPE;
  if ((long long)N * Hl * d * (long long)elem_size(dtype) >= (1LL << 31)) return ULY_ESHAPE;
  return ULY_OK;
}

}  // namespace uly_host
