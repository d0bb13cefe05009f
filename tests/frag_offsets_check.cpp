// Host-side check of the kernels' LDS fragment offsets: for every lane and
// every fragment the kernels read, the XOR form of FragOffsets must give the
// same byte offset as the element-wise RowTile<D>::off of the swizzled tile
// layout (row operands and both transposing reads), for d = 64 and d = 128.
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

int main() {
  const int b64 = check<64>(), b128 = check<128>();
  std::printf("mismatches d=64: %d d=128: %d\n", b64, b128);
  return b64 + b128 == 0 ? 0 : 1;
}
