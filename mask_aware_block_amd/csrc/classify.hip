// Tile classifier: canonical encoding -> exact SKIP / PARTIAL / FULL state of
// every bm x bn tile, compact per-row lists of the tiles to compute, and a
// longest-first order of tile rows.
//
// The skip / full / partial split is what lets the attention kernel avoid the
// cost the FlashMask rebuttal page points at in a token-by-token dense mask:
// fully masked tiles are never loaded and fully visible tiles need no mask.
//
// Exactness on the interval form: canonical runs are disjoint, so the number
// of masked rows of column j inside [r0, r1) is |[r0,r1) & UT_j| + |[r0,r1) &
// LT_j|.  A tile is SKIP iff that equals r1 - r0 for every column, FULL iff it
// is 0 for every column.
#include "internal.h"

namespace fmask {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ inline int32_t overlap(int32_t r0, int32_t r1, int32_t a, int32_t b) {
  int32_t lo = max(r0, a), hi = min(r1, b);
  return hi > lo ? hi - lo : 0;
}

// One thread per tile; threads of a workgroup share kt and read the same columns.
__global__ void __launch_bounds__(256) k_classify_intervals(const int32_t* iv, int32_t nmask,
                                                            int32_t sq, int32_t skv, int32_t bm,
                                                            int32_t bn, int32_t nqt, int32_t nkt,
                                                            uint8_t* state) {
  int64_t total = (int64_t)nmask * nqt * nkt;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int32_t qt = (int32_t)(t % nqt);
    int32_t kt = (int32_t)((t / nqt) % nkt);
    int64_t m = t / ((int64_t)nqt * nkt);
    int32_t r0 = qt * bm, r1 = min(sq, r0 + bm);
    int32_t c0 = kt * bn, c1 = min(skv, c0 + bn);
    const int32_t* col = iv + m * 4 * (int64_t)skv;
    bool all_masked = true, none_masked = true;
    for (int32_t j = c0; j < c1 && (all_masked || none_masked); ++j) {
      int32_t mc = overlap(r0, r1, col[j], col[skv + j]) +
                   overlap(r0, r1, col[2 * (int64_t)skv + j], col[3 * (int64_t)skv + j]);
      all_masked = all_masked && mc == r1 - r0;
      none_masked = none_masked && mc == 0;
    }
    uint8_t st = all_masked ? FMASK_SKIP : (none_masked ? FMASK_FULL : FMASK_PARTIAL);
    state[(m * nqt + qt) * (int64_t)nkt + kt] = st;
  }
}

// The same rule with one wave per (mask, key tile, kQtPerWave query tiles)
// when the tile is 64 keys wide: lane = key column, whose intervals are read
// once.  For a power-of-two tile height every lane computes the tiles its runs
// cover and touch directly and one AND over the wave settles all 16 tiles;
// otherwise per query tile two ballots give "every column fully masked" (SKIP)
// and "no column masked" (FULL).  Lane qt % kQtPerWave keeps that tile's state
// for one store at the end.
constexpr int kQtPerWave = 16;
__global__ void __launch_bounds__(256) k_classify_intervals_cols(const int32_t* iv, int32_t nmask, int32_t sq,
                                                                 int32_t skv, int32_t bm, int32_t nqt, int32_t nkt,
                                                                 uint8_t* state) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int32_t nqg = (nqt + kQtPerWave - 1) / kQtPerWave;
  if (wv >= (int64_t)nmask * nkt * nqg) return;
  const int32_t qg = (int32_t)(wv % nqg);
  const int32_t kt = (int32_t)((wv / nqg) % nkt);
  const int64_t m = wv / ((int64_t)nqg * nkt);
  const int32_t j = kt * 64 + lane;
  const bool col = j < skv;
  const int32_t* c = iv + m * 4 * (int64_t)skv;
  const int32_t us = col ? c[j] : 0, ue = col ? c[skv + j] : 0;
  const int32_t ls = col ? c[2 * (int64_t)skv + j] : 0, le = col ? c[3 * (int64_t)skv + j] : 0;
  // Rows [r0, r1) of a column are all masked iff they lie inside one of its
  // runs (canonical runs neither overlap nor abut), and none is masked iff
  // neither (non-empty) run meets them: comparisons only, combined as lane masks.
  uint8_t mine = FMASK_SKIP;
  const int32_t q0 = qg * kQtPerWave, q1 = min(nqt, q0 + kQtPerWave);
  if ((bm & (bm - 1)) == 0) {
    // Power-of-two tile height: each lane turns its column's two runs into the
    // tiles q0 .. q0 + 15 that they cover entirely (bits 0..15: SKIP needs this
    // for every column) and the tiles they touch (bits 16..31 hold the tiles
    // they leave untouched: FULL needs this for every column); one AND over
    // the wave gives both.  Tile qt holds rows [qt bm, min(sq, (qt + 1) bm)).
    static_assert(kQtPerWave == 16, "two 16-bit tile sets per word");
    const int sh = __builtin_ctz(bm);
    auto span = [&](int lo, int hi) -> uint32_t {  // tiles lo..hi, as bits relative to q0
      const int a = max(lo - q0, 0), b = min(hi - q0 + 1, kQtPerWave);
      return a < b ? ((1u << b) - 1u) & ~((1u << a) - 1u) : 0u;
    };
    auto covered = [&](int s0, int e0) -> uint32_t {  // every row of the tile in [s0, e0)
      if (s0 >= e0) return 0u;
      return span((s0 + bm - 1) >> sh, e0 >= sq ? nqt - 1 : (e0 >> sh) - 1);
    };
    auto touched = [&](int s0, int e0) -> uint32_t {  // some row of the tile in [s0, e0)
      if (s0 >= e0 || s0 >= sq) return 0u;
      return span(s0 >> sh, (min(e0, sq) - 1) >> sh);
    };
    uint32_t w = 0xffffffffu;  // columns past skv leave both sets whole
    if (col) w = (covered(us, ue) | covered(ls, le)) | ((~(touched(us, ue) | touched(ls, le)) & 0xffffu) << 16);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) w &= (uint32_t)__shfl_xor((int)w, o);
    if (lane < kQtPerWave)
      mine = ((w >> lane) & 1u) ? FMASK_SKIP : (((w >> (16 + lane)) & 1u) ? FMASK_FULL : FMASK_PARTIAL);
    if (q0 + lane < q1) state[(m * nqt + q0 + lane) * (int64_t)nkt + kt] = mine;
    return;
  }
  const uint64_t cols = __ballot(col);
  const uint64_t ne_u = __ballot(us < ue), ne_l = __ballot(ls < le);  // non-empty runs
  for (int32_t qt = q0; qt < q1; ++qt) {
    const int32_t r0 = qt * bm, r1 = min(sq, r0 + bm);
    // (one compare per ballot: the masks combine on the scalar unit)
    const uint64_t inside = (__ballot(us <= r0) & __ballot(r1 <= ue)) | (__ballot(ls <= r0) & __ballot(r1 <= le));
    const uint64_t meets = (ne_u & __ballot(us < r1) & __ballot(r0 < ue)) | (ne_l & __ballot(ls < r1) & __ballot(r0 < le));
    const bool all_masked = (inside & cols) == cols;
    const bool none_masked = (meets & cols) == 0ull;
    const uint8_t st = all_masked ? FMASK_SKIP : (none_masked ? FMASK_FULL : FMASK_PARTIAL);
    if (lane == qt - q0) mine = st;
  }
  if (q0 + lane < q1) state[(m * nqt + q0 + lane) * (int64_t)nkt + kt] = mine;
}

// Bitmap form, tiles made of whole 64 x 64 blocks: combine the exact block states.
__global__ void __launch_bounds__(256) k_classify_bitmap(const uint8_t* bstate, int32_t nmask,
                                                         int32_t nbq, int32_t nbk, int32_t bm,
                                                         int32_t bn, int32_t nqt, int32_t nkt,
                                                         uint8_t* state) {
  int64_t total = (int64_t)nmask * nqt * nkt;
  int rb = bm / kBlk, cb = bn / kBlk;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int32_t kt = (int32_t)(t % nkt);
    int32_t qt = (int32_t)((t / nkt) % nqt);
    int64_t m = t / ((int64_t)nqt * nkt);
    bool all_skip = true, all_full = true;
    for (int i = 0; i < rb; ++i) {
      int bi = qt * rb + i;
      if (bi >= nbq) break;
      for (int j = 0; j < cb; ++j) {
        int bj = kt * cb + j;
        if (bj >= nbk) break;
        uint8_t s = bstate[(m * nbq + bi) * (int64_t)nbk + bj];
        all_skip = all_skip && s == FMASK_SKIP;
        all_full = all_full && s == FMASK_FULL;
      }
    }
    state[t] = all_skip ? FMASK_SKIP : (all_full ? FMASK_FULL : FMASK_PARTIAL);
  }
}

// One wave per tile row: stream compaction of the non-SKIP tiles.
__global__ void __launch_bounds__(256) k_tile_lists(const uint8_t* state, int32_t rows, int32_t nkt,
                                                    int32_t* list, int32_t* count) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t* st = state + (int64_t)row * nkt;
  int32_t* out = list + (int64_t)row * nkt;
  int running = 0;
  // the states of up to 512 tiles loaded at once (8 per lane), then compacted
  // 64 at a time
  for (int base0 = 0; base0 < nkt; base0 += 512) {
    uint8_t sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int kt = base0 + 64 * k + lane;
      sv[k] = kt < nkt ? st[kt] : (uint8_t)FMASK_SKIP;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int kt = base0 + 64 * k + lane;
      const bool keep = sv[k] != FMASK_SKIP;
      const uint64_t bal = __ballot(keep);
      const int rank = running + __popcll(bal & ((1ull << lane) - 1ull));
      if (keep) out[rank] = (int32_t)((uint32_t)kt | (sv[k] == FMASK_FULL ? FMASK_LIST_FULL_BIT : 0u));
      running += __popcll(bal);
    }
  }
  for (int i = running + lane; i < nkt; i += 64) out[i] = 0;
  if (lane == 0) count[row] = running;
}

// One wave per tile column (mask m, key tile kt): compaction of the non-SKIP
// query tiles of that column, read from the row-major state table.
__global__ void __launch_bounds__(256) k_tile_cols(const uint8_t* state, int32_t cols, int32_t nqt,
                                                   int32_t nkt, int32_t* list, int32_t* count) {
  int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (col >= cols) return;
  const int m = col / nkt, kt = col % nkt;
  const uint8_t* st = state + (int64_t)m * nqt * nkt + kt;
  int32_t* out = list + (int64_t)col * nqt;
  int running = 0;
  for (int base = 0; base < nqt; base += 64) {
    int qt = base + lane;
    uint8_t s = qt < nqt ? st[(int64_t)qt * nkt] : (uint8_t)FMASK_SKIP;
    bool keep = s != FMASK_SKIP;
    uint64_t bal = __ballot(keep);
    int rank = running + __popcll(bal & ((1ull << lane) - 1ull));
    if (keep) out[rank] = (int32_t)((uint32_t)qt | (s == FMASK_FULL ? FMASK_LIST_FULL_BIT : 0u));
    running += __popcll(bal);
  }
  for (int i = running + lane; i < nqt; i += 64) out[i] = 0;
  if (lane == 0) count[col] = running;
}

// Rank of every tile row within its slice of `seg` consecutive rows (one mask
// slice of the tile table) under (count descending, index ascending), plus the
// slice's first row: the rank is unique, so order[rank] = row is a permutation
// that lists slice 0's rows longest first, then slice 1's, and so on.
// A workgroup ranks 64 rows (lane = row); its four waves count the larger keys
// in four quarters of each 512-key chunk of the slices those rows fall in, and
// the quarters' counts are summed through LDS.
__global__ void __launch_bounds__(256) k_tile_order(const int32_t* count, int32_t rows, int32_t seg,
                                                    int32_t* order) {
  // Row y's key count[y] * 2^32 + (2^32 - 1 - y): the rank of row x is the
  // slice start plus the number of larger keys in its slice.
  __shared__ __attribute__((aligned(16))) uint64_t key[512];
  __shared__ int32_t part[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = blockIdx.x * 64 + lane;
  auto key_of = [](int32_t c, int y) -> uint64_t { return ((uint64_t)(uint32_t)c << 32) | (uint32_t)(~y); };
  const uint64_t kx = x < rows ? key_of(count[x], x) : 0ull;
  const int lo = x / seg * seg, hi = min(lo + seg, rows);
  const int first = blockIdx.x * 64;
  const int last = min(first + 64, rows) - 1;
  const int scan_lo = first / seg * seg, scan_hi = min((last / seg + 1) * seg, rows);
  const bool one_slice = scan_hi - scan_lo <= seg;  // every key scanned is in the slice of every row here
  int rank = 0;
  for (int base = scan_lo; base < scan_hi; base += 512) {
    __syncthreads();
    uint64_t v[2];  // both loads in flight before the stores; padding keys are 0
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int y = base + threadIdx.x + 256 * k;
      v[k] = y < scan_hi ? key_of(count[y], y) : 0ull;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) key[threadIdx.x + 256 * k] = v[k];
    __syncthreads();
    const int lim = min(512, scan_hi - base);
    const int q = (lim + 3) / 4, i0 = w * q, i1 = min(lim, i0 + q);  // this wave's quarter
    if (one_slice) {
#pragma unroll 8
      for (int i = i0; i < i1; ++i) rank += key[i] > kx;
    } else {
#pragma unroll 8
      for (int i = i0; i < i1; ++i) {
        const int y = base + i;
        rank += (key[i] > kx) & (y >= lo) & (y < hi);
      }
    }
  }
  part[w][lane] = rank;
  __syncthreads();
  if (w == 0 && x < rows) order[lo + part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane]] = x;
}

inline int grid_for(int64_t n, int per_block, int cap = 65535 * 16) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

hipError_t launch_classify_intervals(const int32_t* iv, int32_t nmask, int32_t sq, int32_t skv,
                                     int32_t bm, int32_t bn, int32_t nqt, int32_t nkt,
                                     uint8_t* state, hipStream_t s) {
  int64_t total = (int64_t)nmask * nqt * nkt;
  if (total <= 0) return hipSuccess;
  if (bn == 64) {
    const int64_t waves = (int64_t)nmask * nkt * ((nqt + kQtPerWave - 1) / kQtPerWave);
    if ((waves + 3) / 4 <= INT32_MAX) {
      hipLaunchKernelGGL(k_classify_intervals_cols, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, iv, nmask,
                         sq, skv, bm, nqt, nkt, state);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(k_classify_intervals, dim3(grid_for(total, 256)), dim3(256), 0, s, iv, nmask,
                     sq, skv, bm, bn, nqt, nkt, state);
  return hipGetLastError();
}

hipError_t launch_classify_bitmap(const uint8_t* bstate, int32_t nmask, int32_t nbq, int32_t nbk,
                                  int32_t bm, int32_t bn, int32_t nqt, int32_t nkt,
                                  uint8_t* state, hipStream_t s) {
  int64_t total = (int64_t)nmask * nqt * nkt;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_classify_bitmap, dim3(grid_for(total, 256)), dim3(256), 0, s, bstate, nmask,
                     nbq, nbk, bm, bn, nqt, nkt, state);
  return hipGetLastError();
}

hipError_t launch_tile_lists(const uint8_t* state, int32_t rows, int32_t nkt, int32_t* list,
                             int32_t* count, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tile_lists, dim3((rows + 3) / 4), dim3(256), 0, s, state, rows, nkt, list,
                     count);
  return hipGetLastError();
}

hipError_t launch_tile_cols(const uint8_t* state, int32_t nmask, int32_t nqt, int32_t nkt,
                            int32_t* list, int32_t* count, hipStream_t s) {
  const int64_t cols = (int64_t)nmask * nkt;
  if (cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tile_cols, dim3((unsigned)((cols + 3) / 4)), dim3(256), 0, s, state,
                     (int32_t)cols, nqt, nkt, list, count);
  return hipGetLastError();
}

hipError_t launch_tile_order(const int32_t* count, int32_t rows, int32_t seg, int32_t* order,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (seg <= 0 || seg > rows) seg = rows;
  hipLaunchKernelGGL(k_tile_order, dim3((rows + 63) / 64), dim3(256), 0, s, count, rows, seg, order);
  return hipGetLastError();
}

}  // namespace fmask
