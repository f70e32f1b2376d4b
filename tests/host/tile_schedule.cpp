// Host-side check of the grouped FFN's tile-schedule codes: prints, for the
// codes the library picks, the M-tile count of every expert row count up to
// a bound, and the library's class and code decisions for a few shapes.
// Built and run by tests/test_tile_schedule.py; no GPU is used.
#include <cstdio>

#include "common.h"
#include "launch.h"

int main() {
  using namespace moe;
  // shapes: bf16, fp8, E, mean rows per expert, d_model, d_ff
  struct Shape { bool bf16, fp8; int E, rows, d, dff; };
  const Shape shapes[] = {
      {true, false, 128, 1024, 2048, 768},   // capacity-limited, many experts
      {true, false, 32, 1024, 2880, 2880},   // 32 experts
      {true, false, 8, 1024, 4096, 14336},   // 8 experts
      {true, false, 256, 128, 7168, 2048},   // about one tile per expert
      {true, false, 64, 257, 256, 192},      // just above 256 rows per expert
      {true, false, 64, 256, 256, 192},      // exactly 256
      {true, true, 128, 1024, 2048, 768},    // FP8 weights
      {false, false, 128, 1024, 2048, 768},  // fp32 layer
      {true, false, 16, 375, 264, 2112},     // split down projection
  };
  for (const Shape& s : shapes) {
    const bool two = ffn_two_class(s.bf16, s.fp8, s.E, s.rows, s.d, s.dff);
    std::printf("shape %d %d %d %d %d %d two_class %d code %d code2 %d split %d\n", s.bf16, s.fp8,
                s.E, s.rows, s.d, s.dff, two ? 1 : 0, ffn_tile_code(s.bf16, s.rows, s.fp8, two),
                ffn_tile_code2(two), ffn_split_down(s.bf16, s.E, s.rows, s.d, s.dff) ? 1 : 0);
  }
  const int codes[] = {32, 160, 256, kTallTileCode, 160 | kClassSmall, kTallTileCode | kClassLarge,
                       kTallTileCode | kClassSmall, 256 | kClassLarge};
  std::printf("class_rows %d\n", kClassRows);
  for (int c : codes) {
    std::printf("code %d:", c);
    for (int rows = 0; rows <= 3000; ++rows) std::printf(" %d", m_tiles(rows, c));
    std::printf("\n");
  }
  return 0;
}
