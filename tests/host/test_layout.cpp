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

// Extra LDS cycles of one ds_read_b128 (lane l reads 16 bytes at addr[l]) under
// the gfx950 bank model: 64 banks of 4 bytes; lanes served in four groups of
// 16 keyed by (bit 5, bit 4 ^ bit 2) of the lane id.
static int b128_conflicts(const int* addr) {
  int extra = 0;
  for (int g = 0; g < 4; ++g) {
    int cnt[64] = {0};
    int worst = 0;
    for (int l = 0; l < 64; ++l) {
      const int gid = (((l >> 5) & 1) << 1) | (((l >> 4) ^ (l >> 2)) & 1);
      if (gid != g) continue;
      for (int d = 0; d < 4; ++d) {
        const int b = (addr[l] / 4 + d) % 64;
        if (++cnt[b] > worst) worst = cnt[b];
      }
    }
    extra += worst - 1;
  }
  return extra;
}

// Extra cycles of a ds_read_b128 under a second grouping, (bit 2 ^ bit 3,
// bit 2 ^ bit 4) of the lane id, that also fits every measured conflict count
// (the 32x32x16 reads above, and the 16x16x32 reads that conflict under the
// 32x32 key of 128-byte rows but not under the 16x16 key).
static int b128_conflicts_g2(const int* addr) {
  int extra = 0;
  for (int g = 0; g < 4; ++g) {
    int cnt[64] = {0};
    int worst = 0;
    for (int l = 0; l < 64; ++l) {
      const int gid = ((((l >> 2) ^ (l >> 3)) & 1) << 1) | (((l >> 2) ^ (l >> 4)) & 1);
      if (gid != g) continue;
      for (int d = 0; d < 4; ++d) {
        const int b = (addr[l] / 4 + d) % 64;
        if (++cnt[b] > worst) worst = cnt[b];
      }
    }
    extra += worst - 1;
  }
  return extra;
}

// 16x16x32 fragment reads on 128-byte rows: lane l reads row base + l%16,
// logical chunk 4kk + l/16.
template <int MI>
static int frag16_conflicts(int base, int kk) {
  using Z = LdsSwizzle<128, MI>;
  int addr[64];
  for (int l = 0; l < 64; ++l) addr[l] = Z::offset_bytes(base + (l & 15), 4 * kk + (l >> 4));
  return b128_conflicts_g2(addr);
}

static void check_swizzle16() {
  using Z = LdsSwizzle<128, 16>;
  for (int r = 0; r < 256; ++r) {
    std::set<int> seen;
    for (int c = 0; c < 8; ++c) seen.insert(Z::phys_chunk(r, c));
    CHECK((int)seen.size() == 8, "16x16 swizzle not a bijection in row %d", r);
    CHECK(Z::key(r) == Z::key(r & 15), "16x16 key depends on row bits above 3");
  }
  for (int base = 0; base < 256; base += 16)
    for (int kk = 0; kk < 2; ++kk) {
      CHECK(frag16_conflicts<16>(base, kk) == 0, "16x16 fragment-read conflict base %d kk %d", base, kk);
      CHECK(frag16_conflicts<32>(base, kk) > 0, "model should flag the 32x32 key for 16x16 reads");
    }
  // the 32x32 patterns stay conflict-free under this grouping too
  for (int base = 0; base < 256; base += 32)
    for (int kk = 0; kk < 4; ++kk) {
      int addr[64];
      for (int l = 0; l < 64; ++l) addr[l] = LdsSwizzle<128>::offset_bytes(base + (l & 31), 2 * kk + (l >> 5));
      CHECK(b128_conflicts_g2(addr) == 0, "32x32 128-byte reads conflict under the second grouping");
    }
  // direct loads: one wavefront writes 8 whole rows contiguously
  for (int r0 = 0; r0 < 256; r0 += 8) {
    std::set<int> offs;
    for (int l = 0; l < 64; ++l) offs.insert(Z::offset_bytes(r0 + l / 8, Z::logical_chunk(r0 + l / 8, l % 8)));
    CHECK(offs.size() == 64 && *offs.begin() == r0 * 128 && *offs.rbegin() == r0 * 128 + 63 * 16,
          "16x16 direct-load span not contiguous");
  }
}

// Both row swizzles: bijective, fragment reads and direct loads conflict-free.
template <int RowBytes>
void check_swizzle() {
  using Z = LdsSwizzle<RowBytes>;
  const int kc = Z::kChunks;
  CHECK(kc * 16 == RowBytes, "chunks per row");
  for (int r = 0; r < 256; ++r) {
    std::set<int> seen;
    for (int c = 0; c < kc; ++c) seen.insert(Z::phys_chunk(r, c));
    CHECK((int)seen.size() == kc, "swizzle not a bijection in row %d (%d-byte rows)", r, RowBytes);
    for (int c = 0; c < kc; ++c) CHECK(Z::logical_chunk(r, Z::phys_chunk(r, c)) == c, "inverse");
    // the key is a function of the row's low bits only: every 32-row MFMA
    // tile of a stage sees the same keys
    CHECK(Z::key(r) == Z::key(r & 31), "key depends on row bits above 4");
  }
  // fragment reads under the measured gfx950 bank model (64 banks x 4 B; a
  // ds_read_b128 serves the 16 lanes with equal (bit5, bit4^bit2) together):
  // lane l reads row base + l%32, logical chunk 2kk + l/32.
  for (int base = 0; base < 256; base += 32)
    for (int kk = 0; kk < kc / 2; ++kk) {
      int addr[64];
      for (int l = 0; l < 64; ++l) addr[l] = Z::offset_bytes(base + (l & 31), 2 * kk + (l >> 5));
      CHECK(b128_conflicts(addr) == 0, "fragment-read bank conflict base %d kk %d (%d-byte rows)", base, kk,
            RowBytes);
    }
  // direct loads: one wavefront writes 1 KiB = 1024/RowBytes whole rows contiguously
  const int rows = 1024 / RowBytes;
  for (int r0 = 0; r0 < 256; r0 += rows) {
    std::set<int> offs;
    for (int l = 0; l < 64; ++l) offs.insert(Z::offset_bytes(r0 + l / kc, Z::logical_chunk(r0 + l / kc, l % kc)));
    CHECK(offs.size() == 64 && *offs.begin() == r0 * RowBytes && *offs.rbegin() == r0 * RowBytes + 63 * 16,
          "direct-load span not contiguous (%d-byte rows)", RowBytes);
  }
}

// ds_read_b64_tr_b16 as measured on gfx950: in each 16-lane group G, lane
// 4e + j (e, j < 4) names 8 bytes = row e, columns 4j..4j+3 of a 4 x 16 block;
// lane i of the group receives column i.  `img` is LDS as b16 values.
static void tr16_read(const std::vector<int>& img, const int (&addr)[64], int (&out)[64][4]) {
  for (int L = 0; L < 64; ++L) {
    const int G = L / 16, i = L % 16;
    for (int e = 0; e < 4; ++e) out[L][e] = img[(addr[16 * G + 4 * e + i / 4] >> 1) + (i % 4)];
  }
}

// 64-bit LDS reads: conflict-free iff each 32-lane pass touches 64 distinct
// banks; `pairing` 0: passes [0,32) and [32,64); 1: passes by lane bit 4.
static bool b64_conflict_free(const int (&addr)[64], int pairing) {
  for (int pass = 0; pass < 2; ++pass) {
    std::set<int> banks;
    int n = 0;
    for (int l = 0; l < 64; ++l) {
      const int which = pairing == 0 ? (l >> 5) : ((l >> 4) & 1);
      if (which != pass) continue;
      for (int d = 0; d < 2; ++d) banks.insert((addr[l] / 4 + d) % 64);
      n += 2;
    }
    if ((int)banks.size() != n) return false;
  }
  return true;
}

// Transposed tiles: bijective rows, whole-row direct loads, fragment reads that
// deliver the MFMA operand map, conflict-free under both pass pairings.
template <int RowBytes, int MI = 32>
void check_tr_swizzle(int bk) {
  using Z = TrSwizzle<RowBytes, MI>;
  const int W = RowBytes / 2;   // values per row
  for (int k = 0; k < 64; ++k) {
    std::set<int> seen;
    for (int c = 0; c < Z::kChunks; ++c) {
      seen.insert(Z::phys_chunk(k, c));
      CHECK(Z::logical_chunk(k, Z::phys_chunk(k, c)) == c, "tr inverse");
    }
    CHECK((int)seen.size() == Z::kChunks, "tr swizzle not a bijection (%d-byte rows, k %d)", RowBytes, k);
  }
  // direct loads: a 1 KiB span of whole rows, every (row, chunk) once
  for (int s0 = 0; s0 < bk * RowBytes; s0 += 1024) {
    std::set<int> offs;
    for (int l = 0; l < 64; ++l) {
      const int byte = s0 + 16 * l;
      const int k = byte / RowBytes, pc = (byte % RowBytes) / 16;
      offs.insert(Z::offset_bytes(k, 8 * Z::logical_chunk(k, pc)));
    }
    CHECK(offs.size() == 64 && *offs.begin() == s0 && *offs.rbegin() == s0 + 63 * 16, "tr direct-load span");
  }
  // LDS image of a tile whose value at (k, m) is k * 1000 + m
  std::vector<int> img(bk * W);
  for (int k = 0; k < bk; ++k)
    for (int m = 0; m < W; ++m) img[Z::offset_bytes(k, m) / 2] = k * 1000 + m;
  if (MI == 16) {
    // 16x16x32: lane l = 16 g + 4 r + q reads K row 32 kk + 8 g + 4 t + r, values m = mbase + 4 q
    for (int kk = 0; kk < bk / 32; ++kk)
      for (int t = 0; t < 2; ++t)
        for (int mbase = 0; mbase < W; mbase += 16) {
          int addr[64];
          for (int l = 0; l < 64; ++l) {
            const int k = 32 * kk + 8 * (l >> 4) + 4 * t + ((l >> 2) & 3);
            addr[l] = Z::offset_bytes(k, mbase + 4 * (l & 3));
          }
          int got[64][4];
          tr16_read(img, addr, got);
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 4; ++e) {
              const int k = 32 * kk + mfma16::operand_k(l, 4 * t + e), m = mbase + mfma16::operand_row(l);
              CHECK(got[l][e] == k * 1000 + m, "tr16 fragment wrong: rows %d, lane %d, e %d", RowBytes, l, e);
            }
          CHECK(b64_conflict_free(addr, 0), "tr16 read conflicts (pairing 0, %d-byte rows, kk %d t %d m %d)",
                RowBytes, kk, t, mbase);
          CHECK(b64_conflict_free(addr, 1), "tr16 read conflicts (pairing 1, %d-byte rows, kk %d t %d m %d)",
                RowBytes, kk, t, mbase);
        }
    return;
  }
  for (int kk = 0; kk < bk / 16; ++kk)
    for (int t = 0; t < 2; ++t)
      for (int mbase = 0; mbase < W; mbase += 32) {
        int addr[64];
        for (int l = 0; l < 64; ++l) {
          const int r = (l >> 2) & 3, q = l & 3;
          const int k = 16 * kk + 8 * (l >> 5) + 4 * t + r;
          addr[l] = Z::offset_bytes(k, mbase + 16 * ((l >> 4) & 1) + 4 * q);
        }
        int got[64][4];
        tr16_read(img, addr, got);
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 4; ++e) {
            const int k = 16 * kk + mfma32::operand_k(l, 4 * t + e), m = mbase + mfma32::operand_row(l);
            CHECK(got[l][e] == k * 1000 + m, "tr fragment wrong: rows %d, lane %d, e %d", RowBytes, l, e);
          }
        CHECK(b64_conflict_free(addr, 0), "tr read conflicts (pairing 0, %d-byte rows, kk %d t %d m %d)",
              RowBytes, kk, t, mbase);
        CHECK(b64_conflict_free(addr, 1), "tr read conflicts (pairing 1, %d-byte rows, kk %d t %d m %d)",
              RowBytes, kk, t, mbase);
      }
  // the swizzle is needed: unswizzled rows conflict under at least one pairing
  if (RowBytes >= 128) {
    int addr[64];
    for (int l = 0; l < 64; ++l)
      addr[l] = (8 * (l >> 5) + ((l >> 2) & 3)) * RowBytes + 2 * (16 * ((l >> 4) & 1) + 4 * (l & 3));
    CHECK(!(b64_conflict_free(addr, 0) && b64_conflict_free(addr, 1)), "unswizzled tr rows should conflict");
  }
}

// 16-bit output staging: bijection per row; the accumulator writes (16
// lanes of one 4-column group on 16 consecutive rows, 8 bytes each) land on 16
// distinct 16-byte bank groups; the read-back accesses cover contiguous 1 KiB.
template <int RowBytes>
void check_out_swizzle() {
  using Z = OutSwizzle<RowBytes>;
  const int kc = Z::kChunks;
  CHECK(kc * 16 == RowBytes, "out chunks per row");
  for (int r = 0; r < 256; ++r) {
    std::set<int> seen;
    for (int c = 0; c < kc; ++c) {
      seen.insert(Z::phys_chunk(r, c));
      CHECK(Z::logical_chunk(r, Z::phys_chunk(r, c)) == c, "out inverse");
    }
    CHECK((int)seen.size() == kc, "out swizzle not a bijection (%d-byte rows, row %d)", RowBytes, r);
  }
  const int width = RowBytes / 2;                      // 16-bit values per row
  for (int si = 0; si < 8; ++si)
    for (int col4 = 0; col4 < width; col4 += 4) {      // a 4-column group: lanes 16 q .. 16 q + 15
      std::set<int> groups;
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * si + i;
        const int off = Z::offset_bytes(r, col4 >> 3) + 2 * (col4 & 7);
        groups.insert((off % 256) / 16);
      }
      CHECK((int)groups.size() == 16, "out staging write conflict (%d-byte rows, si %d, col %d)", RowBytes, si, col4);
    }
  const int rows_per_access = 1024 / RowBytes;
  for (int p = 0; p < 8; ++p) {
    std::set<int> offs;
    for (int l = 0; l < 64; ++l) {
      const int r = p * rows_per_access + l / kc;
      offs.insert(Z::offset_bytes(r, l % kc));
    }
    CHECK((int)offs.size() == 64 && *offs.begin() == p * 1024 && *offs.rbegin() == p * 1024 + 63 * 16,
          "out read-back access not a contiguous 1 KiB (%d-byte rows, access %d)", RowBytes, p);
  }
}

int main() {
  check_swizzle<64>();
  check_swizzle<128>();
  check_swizzle16();
  check_tr_swizzle<64>(32);
  check_tr_swizzle<128>(64);
  check_tr_swizzle<256>(64);
  check_tr_swizzle<512>(64);
  check_tr_swizzle<128, 16>(64);
  check_tr_swizzle<256, 16>(64);
  check_tr_swizzle<512, 16>(64);
  // the 32x32x16 key would conflict for 16x16x32 reads under the bit-4 pairing
  {
    using Z = TrSwizzle<512, 32>;
    int addr[64];
    for (int l = 0; l < 64; ++l) addr[l] = Z::offset_bytes(8 * (l >> 4) + ((l >> 2) & 3), 4 * (l & 3));
    CHECK(!b64_conflict_free(addr, 1), "32x32 tr key should conflict for 16x16 reads");
  }
  // the model reproduces the measured conflicts of unswizzled rows
  {
    int addr[64];
    for (int l = 0; l < 64; ++l) addr[l] = (l & 31) * 64 + 16 * (l >> 5);
    CHECK(b128_conflicts(addr) > 0, "bank model should flag unswizzled 64-byte rows");
    for (int l = 0; l < 64; ++l) addr[l] = (l & 31) * 128 + 16 * (l >> 5);
    CHECK(b128_conflicts(addr) > 0, "bank model should flag unswizzled 128-byte rows");
  }
  // direct loads: lane l writes byte 16 l of a 1 KiB span
  {
    int addr[64];
    for (int l = 0; l < 64; ++l) addr[l] = 16 * l;
    CHECK(b128_conflicts(addr) == 0, "direct-load span conflicts");
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
    std::set<std::pair<int, int>> cells16, ops16;
    for (int l = 0; l < 64; ++l)
      for (int v = 0; v < mfma16::kAcc; ++v) cells16.insert({mfma16::acc_row(l, v), mfma16::acc_col(l, v)});
    CHECK(cells16.size() == 16 * 16, "mfma16 accumulator map not a bijection");
    for (int l = 0; l < 64; ++l)
      for (int e = 0; e < 8; ++e) ops16.insert({mfma16::operand_row(l), mfma16::operand_k(l, e)});
    CHECK(ops16.size() == 16 * 32, "mfma16 operand map not a bijection");
  }
  // v_permlane16_swap (16-lane rows 1 and 3 of x trade with rows 0 and 2 of y, as probed on
  // gfx950) on the accumulators of two adjacent 16x16 tiles gives the swapped_row/col map
  for (int v = 0; v < mfma16::kAcc; ++v) {
    int x[64][2], y[64][2];   // (row, col) in the 16x32 pair held by lane l
    for (int l = 0; l < 64; ++l) {
      x[l][0] = mfma16::acc_row(l, v), x[l][1] = mfma16::acc_col(l, v);
      y[l][0] = mfma16::acc_row(l, v), y[l][1] = 16 + mfma16::acc_col(l, v);
    }
    int xs[64][2], ys[64][2];
    for (int l = 0; l < 64; ++l) {
      const int row = l >> 4, i = l & 15;
      for (int k = 0; k < 2; ++k) {
        xs[l][k] = (row & 1) == 0 ? x[l][k] : y[16 * (row - 1) + i][k];
        ys[l][k] = (row & 1) == 0 ? x[16 * (row + 1) + i][k] : y[l][k];
      }
    }
    for (int l = 0; l < 64; ++l) {
      CHECK(xs[l][0] == mfma16::swapped_row(l, 0, v) && xs[l][1] == mfma16::swapped_col(l), "swap x lane %d v %d", l, v);
      CHECK(ys[l][0] == mfma16::swapped_row(l, 1, v) && ys[l][1] == mfma16::swapped_col(l), "swap y lane %d v %d", l, v);
    }
  }
  {
    std::set<std::pair<int, int>> cells;
    for (int l = 0; l < 64; ++l)
      for (int t = 0; t < 2; ++t)
        for (int v = 0; v < 4; ++v) cells.insert({mfma16::swapped_row(l, t, v), mfma16::swapped_col(l)});
    CHECK(cells.size() == 16 * 32, "swapped map not a bijection of the 16x32 pair");
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
  for (uint32_t total : {1u, 7u, 8u, 9u, 63u, 64u, 100u, 1024u, 1031u, 4096u}) {
    std::vector<int> hit(total, 0);
    for (uint32_t b = 0; b < total; ++b) {
      uint32_t t = sched::xcd_remap(b, total);
      CHECK(t < total, "xcd_remap out of range total %u", total);
      hit[t]++;
    }
    for (uint32_t t = 0; t < total; ++t) CHECK(hit[t] == 1, "xcd_remap not a bijection total %u", total);
  }
  // the largest grid the C ABI accepts stays in range
  CHECK(sched::xcd_remap(0x7FFFFFFEu, 0x7FFFFFFFu) < 0x7FFFFFFFu, "xcd_remap at the grid limit");
  for (int tm : {1, 3, 4, 5, 32, 33})
    for (int tn : {1, 2, 7, 32})
      for (int gm : {1, 4, 8}) {
        std::set<std::pair<long long, long long>> tiles;
        for (uint32_t t = 0; t < (uint32_t)(tm * tn); ++t) {
          sched::Tile x = sched::grouped_tile(t, tm, tn, gm);
          CHECK(x.m < (uint32_t)tm && x.n < (uint32_t)tn, "grouped_tile out of range");
          tiles.insert({x.m, x.n});
        }
        CHECK((int64_t)tiles.size() == (int64_t)tm * tn, "grouped_tile not a bijection %d %d %d", tm, tn, gm);
      }
  // a contiguous run of 32 ids inside one group covers a 4 x 8 block of a 32 x 32 tile grid
  {
    std::set<long long> ms, ns;
    for (uint32_t t = 0; t < 32; ++t) {
      sched::Tile x = sched::grouped_tile(t, 32, 32, 4);
      ms.insert(x.m);
      ns.insert(x.n);
    }
    CHECK(ms.size() == 4 && ns.size() == 8, "grouped_tile block shape");
  }
  check_out_swizzle<64>();
  check_out_swizzle<128>();
  check_out_swizzle<256>();
  printf("OK %d\n", n_checks);
  return 0;
}
