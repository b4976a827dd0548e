// Host-side checks of layout.hpp (no GPU needed).  Prints "OK <n>" on success,
// "FAIL <what>" and exits 1 on the first failed property.
#include <stdio.h>
#include <stdlib.h>
#include <set>
#include <utility>
#include <vector>

#include "layout.hpp"

using namespace fp16mc;

static int n_checks = 0;
#define CHECK(cond, ...)                              \
  do {                                                \
    ++n_checks;                                       \
    if (!(cond)) {                                    \
      printf("FAIL " __VA_ARGS__);                    \
      printf("\n");                                   \
      exit(1);                                        \
    }                                                 \
  } while (0)

// Bank-group (16-byte unit) of an LDS byte offset for a bank width of `banks` x 4 bytes.
static int bank_group(int byte_off, int banks) { return (byte_off % (banks * 4)) / 16; }

int main() {
  // swizzle: a bijection of the chunks inside every row
  const int kc = lds_swizzle::kChunks;
  for (int r = 0; r < 256; ++r) {
    std::set<int> seen;
    for (int c = 0; c < kc; ++c) seen.insert(lds_swizzle::phys_chunk(r, c));
    CHECK((int)seen.size() == kc, "swizzle not a bijection in row %d", r);
    for (int c = 0; c < kc; ++c) CHECK(lds_swizzle::logical_chunk(r, lds_swizzle::phys_chunk(r, c)) == c, "inverse");
  }
  // fragment reads: lanes 0..31 read rows base..base+31 at one logical chunk.
  // 32 banks: each 8-lane group covers 8 distinct 16-byte bank groups.
  // 64 banks: each 16-lane group covers 16 distinct bank groups.
  for (int base = 0; base < 256; base += 32)
    for (int c = 0; c < kc; ++c) {
      for (int g = 0; g < 4; ++g) {
        std::set<int> bg;
        for (int l = 8 * g; l < 8 * g + 8; ++l) bg.insert(bank_group(lds_swizzle::offset_bytes(base + l, c), 32));
        CHECK(bg.size() == 8, "32-bank conflict base %d chunk %d group %d", base, c, g);
      }
      for (int g = 0; g < 2; ++g) {
        std::set<int> bg;
        for (int l = 16 * g; l < 16 * g + 16; ++l) bg.insert(bank_group(lds_swizzle::offset_bytes(base + l, c), 64));
        CHECK(bg.size() == 16, "64-bank conflict base %d chunk %d group %d", base, c, g);
      }
    }
  // direct loads: one wavefront writes 1 KiB = 16 whole rows contiguously
  for (int r0 = 0; r0 < 256; r0 += 16) {
    std::set<int> offs;
    for (int l = 0; l < 64; ++l) offs.insert(lds_swizzle::offset_bytes(r0 + l / kc, lds_swizzle::logical_chunk(r0 + l / kc, l % kc)));
    CHECK(offs.size() == 64 && *offs.begin() == r0 * lds_swizzle::kRowBytes &&
          *offs.rbegin() == r0 * lds_swizzle::kRowBytes + 63 * 16, "direct-load span not contiguous");
  }
  // MFMA accumulator maps cover the output tile exactly once
  {
    std::set<std::pair<int, int>> cells;
    for (int l = 0; l < 64; ++l)
      for (int v = 0; v < mfma32::kAcc; ++v) cells.insert({mfma32::acc_row(l, v), mfma32::acc_col(l, v)});
    CHECK(cells.size() == 32 * 32, "mfma32 accumulator map not a bijection");
    std::set<std::pair<int, int>> ops;
    for (int l = 0; l < 64; ++l)
      for (int e = 0; e < 8; ++e) ops.insert({mfma32::operand_row(l), mfma32::operand_k(l, e)});
    CHECK(ops.size() == 32 * 16, "mfma32 operand map not a bijection");
  }
  {
    std::set<std::pair<int, int>> cells;
    for (int l = 0; l < 64; ++l)
      for (int v = 0; v < mfma16::kAcc; ++v) cells.insert({mfma16::acc_row(l, v), mfma16::acc_col(l, v)});
    CHECK(cells.size() == 16 * 16, "mfma16 accumulator map not a bijection");
    std::set<std::pair<int, int>> ops;
    for (int l = 0; l < 64; ++l)
      for (int e = 0; e < 8; ++e) ops.insert({mfma16::operand_row(l), mfma16::operand_k(l, e)});
    CHECK(ops.size() == 16 * 32, "mfma16 operand map not a bijection");
  }
  // m8n8: each 32-lane half covers the 8 rows x 4 column pairs once; images are bijections
  for (int num : {1, 2, 4})
    for (int col = 0; col < 2; ++col) {
      std::set<int> offs;
      for (int t = 0; t < num; ++t)
        for (int r = 0; r < 8; ++r)
          for (int c = 0; c < 8; ++c) {
            int o = m8n8::image_offset(col, num, r, c, t);
            CHECK(o >= 0 && o < 64 * num, "image offset out of range");
            offs.insert(o);
          }
      CHECK((int)offs.size() == 64 * num, "image map not a bijection num %d col %d", num, col);
      // row-major words are 4-byte aligned pairs
      if (!col)
        for (int l = 0; l < 32; ++l)
          for (int t = 0; t < num; ++t)
            CHECK(m8n8::image_offset(false, num, m8n8::row(l), 2 * m8n8::col_pair(l), t) % 2 == 0,
                  "row-major fragment word not aligned");
    }
  {
    std::set<std::pair<int, int>> rc;
    for (int l = 0; l < 32; ++l) rc.insert({m8n8::row(l), m8n8::col_pair(l)});
    CHECK(rc.size() == 32, "m8n8 lane map not a bijection");
    CHECK(m8n8::row(32) == 0 && m8n8::half_of_wave(32) == 1, "second half of the wavefront");
  }
  // scheduler: xcd_remap and grouped_tile are bijections
  for (int64_t total : {1, 7, 8, 9, 63, 64, 100, 1024, 1031, 4096}) {
    std::vector<int> hit(total, 0);
    for (int64_t b = 0; b < total; ++b) {
      int64_t t = sched::xcd_remap(b, total);
      CHECK(t >= 0 && t < total, "xcd_remap out of range total %lld", (long long)total);
      hit[t]++;
    }
    for (int64_t t = 0; t < total; ++t) CHECK(hit[t] == 1, "xcd_remap not a bijection total %lld", (long long)total);
  }
  for (int tm : {1, 3, 4, 5, 32, 33})
    for (int tn : {1, 2, 7, 32})
      for (int gm : {1, 4, 8}) {
        std::set<std::pair<long long, long long>> tiles;
        for (int64_t t = 0; t < (int64_t)tm * tn; ++t) {
          sched::Tile x = sched::grouped_tile(t, tm, tn, gm);
          CHECK(x.m >= 0 && x.m < tm && x.n >= 0 && x.n < tn, "grouped_tile out of range");
          tiles.insert({x.m, x.n});
        }
        CHECK((int64_t)tiles.size() == (int64_t)tm * tn, "grouped_tile not a bijection %d %d %d", tm, tn, gm);
      }
  // a contiguous run of 32 ids inside one group covers a 4 x 8 block of a 32 x 32 tile grid
  {
    std::set<long long> ms, ns;
    for (int64_t t = 0; t < 32; ++t) {
      sched::Tile x = sched::grouped_tile(t, 32, 32, 4);
      ms.insert(x.m);
      ns.insert(x.n);
    }
    CHECK(ms.size() == 4 && ns.size() == 8, "grouped_tile block shape");
  }
  printf("OK %d\n", n_checks);
  return 0;
}
