// Internal declarations shared by the libfmask translation units (not part of
// the C ABI).  Kernels are written for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "fmask.h"

namespace fmask {

constexpr int kBlk = FMASK_BLOCK;  // 64: bitmap granularity
constexpr int kXcds = 8;           // MI355X: 8 XCDs, workgroups dealt round-robin

// ---------------------------------------------------------------- encoder
constexpr int kSegInline = 64;

struct SegParams {
  int32_t family;
  int32_t sq, skv;
  const int32_t* cu;  // device copy of cu_seg, n_seg + 1 entries (more than kSegInline segments)
  int32_t n_seg;
  int32_t cu_inline[kSegInline + 1];  // cu_seg itself, up to kSegInline segments (no copy)
  int64_t pre, next;  // band, clamped by the host to +-(sq + skv + 1)
  int32_t tree_prefix;
  const int32_t* tree_hi;  // per draft node: last descendant (interval-form tree)
  // varlen: device copies of cumulative key lengths, modes and prefix widths
  const int32_t* cu_k;
  const int32_t* mode;
  const int32_t* prefix;
};

hipError_t launch_encode_family_intervals(const SegParams& p, int32_t* iv, hipStream_t s);
hipError_t launch_encode_raw_intervals(const int32_t* raw, int32_t nmask, int32_t sq, int32_t skv,
                                       int32_t* iv, hipStream_t s);
// *x = 0 by a one-thread kernel (a fill a captured HIP graph replays correctly).
hipError_t launch_zero_int(int32_t* x, hipStream_t s);
hipError_t launch_tree_hi(const int32_t* parent, int32_t n, int32_t* hi, hipStream_t s);

// Source of the 64-bit row words of a 64 x 64 block, for the bitmap encoder.
struct BitmapSrc {
  int32_t kind;  // 0 = caller bitmap, 1 = tree, 2 = dense bytes
  int32_t nmask, nbq, nbk;
  int32_t sq, skv;
  // caller bitmap
  const uint8_t* state;
  const int32_t* index;
  const uint64_t* bits;
  int64_t pool_n;
  int32_t force_diag;
  // tree
  int32_t tree_prefix, tree_n;
  const int32_t* parent;
  // dense (kind 2): uint8 [nmask][sq][skv], nonzero = visible; dense_vec: rows
  // 16-byte aligned (skv % 16 == 0 and an aligned base), read 16 bytes at a time
  const uint8_t* dense;
  int32_t dense_vec;
};

struct BitmapOut {
  uint8_t* state;       // [nmask][nbq][nbk]
  int32_t* index;       // same
  uint64_t* bits;       // [cap][64]
  int64_t cap;
  int32_t* row_count;   // [nmask * nbq]
  int32_t* row_offset;  // [nmask * nbq]
  int32_t* pool_count;  // scalar
};

hipError_t launch_encode_bitmap(const BitmapSrc& src, const BitmapOut& out, hipStream_t s);
// Dense uint8 masks -> canonical intervals; *bad (zeroed here) becomes nonzero
// if some column has more than two masked runs.
// Dense mask -> canonical intervals.  Rows are split into dense_groups()
// groups so that enough workgroups run; with more than one group `ws` holds
// dense_ws_bytes() of partial runs.
// Columns per workgroup strip: 128 where 16-byte row loads are possible
// (whole 128-byte lines per wave), else 64.
constexpr int dense_strip(bool row_loads) { return row_loads ? 128 : 64; }
inline int32_t dense_groups(int64_t nmask, int32_t sq, int32_t skv) {
  const int64_t strips = nmask * ((skv + 127) / 128);
  if (strips <= 0) return 1;
  const int64_t want = (256 + strips - 1) / strips;  // about 256 workgroups of 16 waves (128-column strips)
  const int64_t most = ((int64_t)sq + 1023) / 1024;  // at least 1024 rows per group
  return (int32_t)std::max<int64_t>(1, std::min(want, most));
}
inline size_t dense_ws_bytes(int64_t nmask, int32_t sq, int32_t skv) {
  const int32_t g = dense_groups(nmask, sq, skv);
  return g > 1 ? (size_t)nmask * g * skv * 20 : 0;  // one 20-byte record of runs per (mask, group, column)
}
hipError_t launch_encode_dense_intervals(const uint8_t* dense, int32_t nmask, int32_t sq, int32_t skv,
                                         void* ws, int32_t* iv, int32_t* bad, hipStream_t s);

hipError_t launch_encode_selected(const int32_t* sel, int32_t nb, int32_t sq, int32_t n,
                                  int32_t nblk, int32_t* list, int32_t* count, hipStream_t s);

// ---------------------------------------------------------------- classifier
hipError_t launch_classify_intervals(const int32_t* iv, int32_t nmask, int32_t sq, int32_t skv,
                                     int32_t bm, int32_t bn, int32_t nqt, int32_t nkt,
                                     uint8_t* state, hipStream_t s);
hipError_t launch_classify_bitmap(const uint8_t* bstate, int32_t nmask, int32_t nbq, int32_t nbk,
                                  int32_t bm, int32_t bn, int32_t nqt, int32_t nkt,
                                  uint8_t* state, hipStream_t s);
hipError_t launch_tile_lists(const uint8_t* state, int32_t rows, int32_t nkt, int32_t* list,
                             int32_t* count, hipStream_t s);
hipError_t launch_tile_cols(const uint8_t* state, int32_t nmask, int32_t nqt, int32_t nkt,
                            int32_t* list, int32_t* count, hipStream_t s);
// order[] of `rows` tile rows: slices of `seg` rows in turn, each longest first
hipError_t launch_tile_order(const int32_t* count, int32_t rows, int32_t seg, int32_t* order,
                             hipStream_t s);

// ---------------------------------------------------------------- attention
struct TileAttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t b, hq, hkv, group;  // group = hq / hkv
  int32_t sq, skv;
  float scale;
  // tile table
  const int32_t* list;
  const int32_t* count;
  const int32_t* order;
  int32_t nqt, nkt, bm, bn;
  int32_t mb, mh;      // distinct masks along batch / heads
  int32_t expand;      // (b, h) pairs per tile row
  int32_t n_items;     // tile rows * expand
  int32_t set_major;   // items dealt to the XCDs by (K/V head, batch) set (o3 kernel)
  // mask
  int32_t kind;        // FMASK_ENC_INTERVALS or FMASK_ENC_BITMAP
  const int32_t* iv;   // [mb][mh][4][skv]
  const uint8_t* bstate;
  const int32_t* bindex;
  const uint64_t* bbits;
  int64_t pool_cap;    // entries of bbits
  int32_t nbq, nbk;
};

hipError_t launch_attn_tile_bf16(const TileAttnParams& p, int32_t d, hipStream_t s);
hipError_t launch_attn_tile_f32(const TileAttnParams& p, int32_t d, hipStream_t s);
hipError_t launch_attn_o3_bf16(const TileAttnParams& p, int32_t d, hipStream_t s);
hipError_t launch_attn_pair_bf16(const TileAttnParams& p, int32_t d, hipStream_t s);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ws;           // [b][hq][sq] x {D_i, LSE_i log2(e) (+inf for empty rows)}
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t b, hq, hkv, group;
  int32_t sq, skv;
  float scale;
  const int32_t* list;
  const int32_t* count;
  const int32_t* order;
  const int32_t* col_list;
  const int32_t* col_count;
  const int32_t* col_order;
  int32_t nqt, nkt, bm, bn;
  int32_t mb, mh;
  int32_t kind;             // FMASK_ENC_INTERVALS or FMASK_ENC_BITMAP
  const int32_t* iv;        // INTERVALS: [mb][mh][4][skv]
  const uint8_t* bstate;    // BITMAP: [mb][mh][nbq][nbk] 64x64 block states
  const int32_t* bindex;    // BITMAP: pool entry of each PARTIAL block
  const uint64_t* bbits;    // BITMAP: [pool][64] row words (bit c: key 64 bj + c)
  int32_t nbq, nbk;
};

hipError_t launch_attn_bwd_bf16(const BwdParams& p, int32_t d, hipStream_t s);

struct SelAttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs[3], ks[3], vs[3], os[3];
  int32_t b, hq, hkv, group;
  int32_t sq, skv;
  float scale;
  const int32_t* list;   // [mb][sq][n]
  const int32_t* count;  // [mb][sq]
  int32_t n, cells, mb;
};

// nsplit > 1: each query's list is split over nsplit workgroups whose partial
// states go to ws (selected_split_ws_floats floats) and are merged afterwards.
hipError_t launch_attn_selected_bf16(const SelAttnParams& p, int32_t d, int32_t nsplit, float* ws,
                                     hipStream_t s);
bool selected_group_supported(int32_t group);
size_t selected_split_ws_floats(const SelAttnParams& p, int32_t d, int32_t nsplit);

// Block-major form of the selected-key forward: workspace pieces (byte offsets)
// for the block index, the per-(batch, query, entry, head) partial states
// and their bf16 outputs.
struct BlkLayout {
  int32_t nblk = 0;
  size_t hist = 0, off = 0, inv = 0, pm = 0, po = 0, total = 0;
};
BlkLayout selected_blocks_layout(const SelAttnParams& p, int32_t d);
hipError_t launch_attn_selected_blocks_bf16(const SelAttnParams& p, int32_t d, void* ws, hipStream_t s);

}  // namespace fmask
