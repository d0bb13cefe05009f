// Host-side check of the kernels' LDS fragment offsets: for every lane and
// every fragment the kernels read, the XOR form of FragOffsets must give the
// same byte offset as the element-wise RowTile<D>::off of the swizzled tile
// layout (row operands and both transposing reads), for d = 64 and d = 128.
// For the natural-order transposing reads (NatTrOffsets) it also emulates
// the read itself (in each group of 16 lanes, lane i receives element i % 4
// of the 8-byte chunks addressed by lanes 4m + i / 4, m = 0..3) and checks
// that lane l ends up with column 32 cb + l % 32 of rows 16 j + 8 (l / 32) +
// (0..7), the order of a 16-byte read of a K-contiguous operand.
// Built for the host only and run by tests/test_frag_offsets_cpu.py.
#include <cstdio>

#include "common.h"

using namespace uly;

template <int D>
static int check() {
  int bad = 0;
  for (int lane = 0; lane < 64; ++lane) {
    FragOffsets<D> fo;
    fo.init(lane);
    const int half = lane >> 5, l32 = lane & 31, p = lane & 15;
    for (int rb = 0; rb < 4; ++rb)
      for (int kk = 0; kk < D / 16; ++kk)
        if (fo.row_frag(rb, kk) != 2u * (uint32_t)RowTile<D>::off(32 * rb + l32, 16 * kk + 8 * half)) ++bad;
    for (int j = 0; j < 8; ++j)
      for (int cb = 0; cb < D / 32; ++cb) {
        const int row = 16 * j + 4 * half + (p >> 2);
        const int col = 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (p & 3);
        const uint32_t x = (uint32_t)cb << 6, rows = (uint32_t)(j * 32 * D);
        if ((fo.tr_lo ^ x) + rows != 2u * (uint32_t)RowTile<D>::off(row, col)) ++bad;
        if ((fo.tr_hi ^ x) + rows != 2u * (uint32_t)RowTile<D>::off(row + 8, col)) ++bad;
      }
  }
  return bad;
}

// (row, col) of the element at a byte offset of a RowTile<D> tile
template <int D>
static void element_at(uint32_t byte, int& row, int& col) {
  const int e = (int)(byte / 2u);
  row = e / D;
  const int within = e % D;
  const int phys_chunk = within / 8;
  col = ((phys_chunk ^ RowTile<D>::chunk_key(row)) << 3) | (within & 7);
}

template <int D>
static int check_natural() {
  int bad = 0;
  for (int j = 0; j < 4; ++j)
    for (int cb = 0; cb < D / 32; ++cb)
      for (int which = 0; which < 2; ++which) {
        uint32_t addr[64];
        for (int lane = 0; lane < 64; ++lane) {
          NatTrOffsets<D> no;
          no.init(lane);
          addr[lane] = ((which ? no.hi : no.lo) ^ ((uint32_t)cb << 6)) + (uint32_t)(j * 32 * D);
        }
        for (int lane = 0; lane < 64; ++lane) {
          const int g0 = lane & ~15, i = lane & 15;
          for (int m = 0; m < 4; ++m) {
            int row, col;
            element_at<D>(addr[g0 + 4 * m + i / 4] + 2u * (uint32_t)(i % 4), row, col);
            const int want_row = 16 * j + 8 * (lane >> 5) + 4 * which + m;
            const int want_col = 32 * cb + (lane & 31);
            if (row != want_row || col != want_col) ++bad;
          }
        }
      }
  return bad;
}

int main() {
  const int b64 = check<64>(), b128 = check<128>();
  std::printf("mismatches d=64: %d d=128: %d\n", b64, b128);
  const int n64 = check_natural<64>(), n128 = check_natural<128>();
  std::printf("natural-order transposing reads, mismatches d=64: %d d=128: %d\n", n64, n128);
  return b64 + b128 + n64 + n128 == 0 ? 0 : 1;
}
