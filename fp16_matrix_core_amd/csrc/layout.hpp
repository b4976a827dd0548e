// layout.hpp -- index maps of the gfx950 data path, as constexpr functions
// usable from host and device code.
//
//   LdsSwizzle    16-byte chunk placement inside the 64- or 128-byte LDS
//                 rows that hold a 32- or 64-element fp16 K slice of an
//                 operand tile.
//   mfma32        lane maps of v_mfma_f32_32x32x16_f16.
//   mfma16        lane maps of v_mfma_f32_16x16x32_f16.
//   m8n8          the 8x8 b16 matrix fragment of the warp-collective matrix
//                 load/store, mapped onto 64-lane wavefronts.
//
// These replace the lane tables that the pages express as TileLayouts for
// m16n8k16 and ldmatrix; they are checked on the host (bijectivity, bank
// spread) and on the GPU by the identity and permutation products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define FP16MC_HD __host__ __device__

namespace fp16mc {

// ---------------------------------------------------------------------------
// LDS swizzles.  A row of an operand tile in LDS holds one K slice of fp16:
// 64 bytes (BK = 32, 4 chunks of 16 bytes) or 128 bytes (BK = 64, 8 chunks).
// Logical chunk c of row r is stored at physical chunk c ^ key(r):
//   64-byte rows   key(r) = (r >> 2) & 3
//   128-byte rows  key(r) = (r & 7) ^ ((r >> 3) & 1)           (32x32x16 reads)
//                  key(r) = r0 | r3 << 1 | r1 << 2              (16x16x32 reads)
// with ri = bit i of r.
// Bank model (measured on gfx950 with collision probes and the SQ bank-
// conflict counter): LDS has 64 banks of 4 bytes, and a ds_read_b128 is
// served 16 lanes at a time, the four groups being the lanes with equal
// (bit 5, bit 4 ^ bit 2) of the lane id -- e.g. lanes {0-3, 8-11, 20-23,
// 28-31}.  Within a group no two lanes may touch the same bank.  Both keys
// make the 32x32x16 fragment reads (lane l reads row l%32, chunk
// 2kk + l/32) conflict-free; the direct loads write whole rows as one
// contiguous kilobyte per wavefront (lane l at byte 16 l), which never
// conflicts.  That lane grouping does not hold for every pattern: the
// 16x16x32 reads (row l%16, chunk 4kk + l/16), which it predicts to be
// conflict-free under the 32x32 key, measured about 4 conflict cycles per
// read (SQ_LDS_BANK_CONFLICT, in the GEMM and in a probe); the 16x16 key
// above measured none (as did r0<<0|r3<<1|r1<<2 variants with r0 or r0^r1
// mixed in), so 16x16 tiles use it.
// The XOR keeps the map a bijection inside each row.
// ---------------------------------------------------------------------------
template <int RowBytes, int MI = 32>
struct RowSwizzle;

template <>
struct RowSwizzle<64, 32> {
  static constexpr int kRowBytes = 64;
  static constexpr int kChunks = 4;
  FP16MC_HD static constexpr int key(int row) { return (row >> 2) & 3; }
};

template <>
struct RowSwizzle<128, 32> {
  static constexpr int kRowBytes = 128;
  static constexpr int kChunks = 8;
  FP16MC_HD static constexpr int key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
};

template <>
struct RowSwizzle<128, 16> {
  static constexpr int kRowBytes = 128;
  static constexpr int kChunks = 8;
  FP16MC_HD static constexpr int key(int row) {
    return (row & 1) | (((row >> 3) & 1) << 1) | (((row >> 1) & 1) << 2);
  }
};

// MI: the matrix instruction whose fragments are read (32: 32x32x16, 16: 16x16x32).
template <int RowBytes, int MI = 32>
struct LdsSwizzle : RowSwizzle<RowBytes, MI> {
  using Base = RowSwizzle<RowBytes, MI>;
  FP16MC_HD static constexpr int phys_chunk(int row, int chunk) { return chunk ^ Base::key(row); }
  // inverse map (the XOR is its own inverse): which logical chunk sits at a physical one
  FP16MC_HD static constexpr int logical_chunk(int row, int phys) { return phys ^ Base::key(row); }
  FP16MC_HD static constexpr int offset_bytes(int row, int chunk) {
    return row * Base::kRowBytes + (phys_chunk(row, chunk) << 4);
  }
};

// ---------------------------------------------------------------------------
// Transposed operand tiles.  An operand stored with M (or N) contiguous is
// staged as it lies in memory: LDS row k holds the tile's RowBytes/2 values
// of K index k.  A matrix-instruction fragment needs 8 consecutive K of one
// M, which ds_read_b64_tr_b16 delivers: in each 16-lane group, lane 4r + q
// names 8 bytes (4 values) of "row" r of a 4 x 16 block and lane i receives
// column i of that block (measured on gfx950).  Lane l = 16 g + 4 r + q of a
// 32x32x16 fragment read takes LDS row k0 + r with k0 = 8 (l / 32) (+4 for
// the second half of the 8 K values) and the 4 values at m = 16 (g % 2) + 4 q;
// of a 16x16x32 one, row 8 g + r (+4) and the values at m = 4 q.
//
// Chunk c of row k is stored at physical chunk c ^ key(k), with
//   64-byte rows    key = 2 b
//   128-byte rows   key = 4 ((k >> 1) & 1) + 2 b
//   >= 256 bytes    key = 4 (k & 3) + 2 b   (low 4 chunk bits)
// where b = bit 3 of k for 32x32x16 fragments and bit 3 ^ bit 4 of k for
// 16x16x32 ones (MI = 16: lane l = 16 g + 4 r + q reads K row 8 g + r, so
// the lanes of a 32-lane pass differ in K-row bit 3 or bit 4).  The 32 lanes
// served together -- lanes [0, 32) and [32, 64), or lanes with equal bit 4 --
// then touch 64 distinct banks (tests/host simulates both pairings).  The
// key uses only K-row bits that are constant across a fragment's K steps
// (0, 1 and 3, and 4 for MI = 16), i.e. it is a per-lane constant of a
// fragment read.  Direct loads fill whole rows as contiguous 1 KiB spans, as
// for K-contiguous tiles.
// ---------------------------------------------------------------------------
template <int RowBytes, int MI = 32>
struct TrSwizzle {
  static_assert(RowBytes == 64 || RowBytes == 128 || (RowBytes >= 256 && RowBytes % 256 == 0),
                "transposed tiles are 32, 64 or a multiple of 128 values wide");
  static_assert(MI == 32 || MI == 16, "32x32x16 or 16x16x32 fragments");
  static constexpr int kRowBytes = RowBytes;
  static constexpr int kChunks = RowBytes / 16;
  FP16MC_HD static constexpr int key(int k) {
    return RowBytes == 64    ? 2 * kbit(k)
           : RowBytes == 128 ? 4 * ((k >> 1) & 1) + 2 * kbit(k)
                             : 4 * (k & 3) + 2 * kbit(k);
  }
  FP16MC_HD static constexpr int kbit(int k) { return MI == 16 ? ((k >> 3) ^ (k >> 4)) & 1 : (k >> 3) & 1; }
  FP16MC_HD static constexpr int phys_chunk(int k, int chunk) { return chunk ^ key(k); }
  FP16MC_HD static constexpr int logical_chunk(int k, int phys) { return phys ^ key(k); }
  // byte offset of element m of row k
  FP16MC_HD static constexpr int offset_bytes(int k, int m) {
    return k * RowBytes + (phys_chunk(k, m >> 3) << 4) + 2 * (m & 7);
  }
};

// ---------------------------------------------------------------------------
// 16-bit output tiles staged in LDS.  Row r of a wave tile of 16-bit values
// fills RowBytes (64, 128 or 256) bytes; its 16-byte chunk c sits at
// physical chunk c ^ key(r) with key(r) = (r / (256 / RowBytes)) mod
// (RowBytes / 16).  The accumulator writes put the 16 lanes of one 4-column
// group on 16 consecutive rows at one logical chunk: the rows that share a
// 256-byte bank window (256 / RowBytes of them) differ in their window
// offset, the others in their key, so the 16 land on 16 different 16-byte
// bank groups.  Reading back, the lanes of a row read its chunks in order:
// each 1 KiB access covers contiguous rows.
// ---------------------------------------------------------------------------
template <int RowBytes>
struct OutSwizzle {
  static_assert(RowBytes == 64 || RowBytes == 128 || RowBytes == 256, "rows of 32, 64 or 128 16-bit values");
  static constexpr int kRowBytes = RowBytes;
  static constexpr int kChunks = RowBytes / 16;
  FP16MC_HD static constexpr int key(int row) { return (row / (256 / RowBytes)) & (kChunks - 1); }
  FP16MC_HD static constexpr int phys_chunk(int row, int chunk) { return chunk ^ key(row); }
  FP16MC_HD static constexpr int logical_chunk(int row, int phys) { return phys ^ key(row); }
  FP16MC_HD static constexpr int offset_bytes(int row, int chunk) {
    return row * RowBytes + (phys_chunk(row, chunk) << 4);
  }
};

// ---------------------------------------------------------------------------
// v_mfma_f32_32x32x16_f16: D(32x32) += X(32x16) * Y(16x32), fp16 in, fp32 acc.
// Operands: lane l supplies 8 fp16 of X row (l % 32), and 8 fp16 of Y column
// (l % 32), both at k = 8*(l / 32) + e, e in [0, 8).
// Accumulator: 16 fp32 per lane; element v of lane l is
// D[8*(v/4) + 4*(l/32) + v%4][l % 32].
// ---------------------------------------------------------------------------
namespace mfma32 {
constexpr int kM = 32, kN = 32, kK = 16, kAcc = 16;
FP16MC_HD constexpr int operand_row(int lane) { return lane & 31; }
FP16MC_HD constexpr int operand_k(int lane, int e) { return 8 * (lane >> 5) + e; }
FP16MC_HD constexpr int acc_row(int lane, int v) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
FP16MC_HD constexpr int acc_col(int lane, int /*v*/) { return lane & 31; }
}  // namespace mfma32

// ---------------------------------------------------------------------------
// v_mfma_f32_16x16x32_f16: D(16x16) += X(16x32) * Y(32x16), the same rate per
// cycle as the 32x32 form with half the accumulator per instruction.
// Operands: lane l supplies 8 fp16 of X row (l % 16), and 8 fp16 of Y column
// (l % 16), both at k = 8*(l / 16) + e, e in [0, 8).
// Accumulator: 4 fp32 per lane; element v of lane l is D[4*(l/16) + v][l % 16].
// ---------------------------------------------------------------------------
namespace mfma16 {
constexpr int kM = 16, kN = 16, kK = 32, kAcc = 4;
FP16MC_HD constexpr int operand_row(int lane) { return lane & 15; }
FP16MC_HD constexpr int operand_k(int lane, int e) { return 8 * (lane >> 4) + e; }
FP16MC_HD constexpr int acc_row(int lane, int v) { return 4 * (lane >> 4) + v; }
FP16MC_HD constexpr int acc_col(int lane, int /*v*/) { return lane & 15; }
// v_permlane16_swap_b32 x, y trades 16-lane rows 1 and 3 of x with rows 0
// and 2 of y.  Applied to element v of two horizontally adjacent tiles (the
// left one's register as x), register t (0: x, 1: y), element v of lane l
// then holds row swapped_row(l, t, v), column swapped_col(l) of the 16x32
// pair: 32 consecutive columns of one row per half-wavefront.
FP16MC_HD constexpr int swapped_row(int lane, int t, int v) { return 4 * t + v + 8 * (lane >> 5); }
FP16MC_HD constexpr int swapped_col(int lane) { return lane & 31; }
}  // namespace mfma16

// ---------------------------------------------------------------------------
// m8n8 fragment of the matrix load/store: over a 32-lane group, lane l holds
// row l/4 and the column pair 2*(l%4), 2*(l%4)+1 of every tile, one 32-bit
// word per tile (even column in the low half).  A 64-lane wavefront carries
// two such groups: lanes [0,32) and [32,64).
// Shared-side images (in b16 units, per group of `num` tiles):
//   row-major     r*8*num + 8*t + c      (row stride p = 8*num)
//   column-major  (8*t + c)*8 + r        (column stride p = 8)
// ---------------------------------------------------------------------------
namespace m8n8 {
FP16MC_HD constexpr int row(int lane) { return (lane & 31) >> 2; }
FP16MC_HD constexpr int col_pair(int lane) { return lane & 3; }
FP16MC_HD constexpr int half_of_wave(int lane) { return lane >> 5; }
FP16MC_HD constexpr int image_offset(bool col_major, int num, int r, int c, int t) {
  return col_major ? (8 * t + c) * 8 + r : r * 8 * num + 8 * t + c;
}
}  // namespace m8n8

// ---------------------------------------------------------------------------
// Workgroup -> output tile.  Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs, each with its own L2.  xcd_remap gives each
// XCD a contiguous range of logical tile ids (a bijection for any count);
// grouped_tile then orders a problem's tiles in column strips of `group_m`
// tile rows so a contiguous id range covers a compact block of the output
// and its A and B panels are reused from that XCD's L2.
// ---------------------------------------------------------------------------
namespace sched {
// 32-bit arithmetic: grids are limited to fewer than 2^31 workgroups, and
// 64-bit integer division is a long instruction sequence on the GPU.
constexpr uint32_t kXcds = 8;
FP16MC_HD constexpr uint32_t xcd_remap(uint32_t bid, uint32_t total) {
  const uint32_t q = total / kXcds, r = total % kXcds;
  const uint32_t x = bid % kXcds, j = bid / kXcds;
  return x * q + (x < r ? x : r) + j;
}
struct Tile {
  uint32_t m, n;
};
FP16MC_HD constexpr Tile grouped_tile(uint32_t t, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m) {
  const uint32_t per_group = group_m * tiles_n;
  const uint32_t g = t / per_group;
  const uint32_t first_m = g * group_m;
  const uint32_t rows = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const uint32_t in_group = t - g * per_group;
  return Tile{first_m + in_group % rows, in_group / rows};
}
}  // namespace sched

}  // namespace fp16mc
