// Mask encoder kernels: mask-family parameters -> canonical compressed forms.
//
// * Interval form: per key column j the masked query rows, as at most two
//   maximal runs UT = [UTS, UTE) and LT = [LTS, LTE) (the per-key-column
//   lower/upper-triangle start/end encoding of FlashMask, as the FlashMask
//   rebuttal page's method uses it).  Every interval family has a single
//   contiguous visible row range per column, so the kernel computes that range
//   [vlo, vhi) and writes its complement canonically.
// * Bitmap form: 64 x 64 blocks (Binary Block Masking) with exact states and a
//   compact pool of 64 row words per PARTIAL block, in row-major block order.
// * Selected-key lists (llama.cpp selected-key PR): valid, distinct, ascending.
#include <algorithm>

#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

// Canonical (UTS, UTE, LTS, LTE) of a column whose visible rows are [vlo, vhi).
__device__ inline void store_visible_range(int32_t* iv, int64_t skv, int64_t j, int64_t vlo,
                                           int64_t vhi, int32_t sq) {
  if (vlo < 0) vlo = 0;
  if (vhi > sq) vhi = sq;
  int32_t uts = 0, ute = 0, lts = sq, lte = sq;
  if (vlo >= vhi) {
    ute = sq;  // everything masked: one run starting at row 0
  } else {
    if (vlo > 0) ute = (int32_t)vlo;
    if (vhi < sq) lts = (int32_t)vhi;
  }
  iv[j] = uts;
  iv[skv + j] = ute;
  iv[2 * skv + j] = lts;
  iv[3 * skv + j] = lte;
}

// Largest s in [0, n_seg) with cu[s] <= pos.
__device__ inline int segment_of(const int32_t* cu, int n_seg, int64_t pos) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void k_family_intervals(SegParams p, int32_t* iv) {
  // segment starts: in the arguments when few, else the device copy (varlen
  // always uses its device copies)
  const int32_t* cu = (p.family != FMASK_VARLEN && p.n_seg <= kSegInline) ? p.cu_inline : p.cu;
  for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < p.skv;
       j += (int64_t)gridDim.x * blockDim.x) {
    int64_t vlo = 0, vhi = p.sq;
    switch (p.family) {
      case FMASK_CAUSAL:  // j <= i
        vlo = j;
        break;
      case FMASK_CAUSAL_BOTTOM_RIGHT:  // j <= i + skv - sq
        vlo = j - ((int64_t)p.skv - p.sq);
        break;
      case FMASK_DOCUMENT: {
        int s = segment_of(cu, p.n_seg, j);
        vlo = cu[s];
        vhi = cu[s + 1];
        break;
      }
      case FMASK_CAUSAL_DOCUMENT: {
        int s = segment_of(cu, p.n_seg, j);
        vlo = j;
        vhi = cu[s + 1];
        break;
      }
      case FMASK_SHARED_QUESTION: {  // question columns: every later row; answers: own answer
        int s = segment_of(cu, p.n_seg, j);
        vlo = j;
        vhi = (s == 0) ? p.sq : cu[s + 1];
        break;
      }
      case FMASK_BAND: {  // r - pre <= j <= r + next with r = i + skv - sq
        int64_t off = (int64_t)p.skv - p.sq;
        vlo = j - p.next - off;
        vhi = j + p.pre - off + 1;
        break;
      }
      case FMASK_VARLEN: {  // the key's segment s: its query rows, under the segment's mode
        const int s = segment_of(p.cu_k, p.n_seg, j);
        const int64_t qs = p.cu[s], qe = p.cu[s + 1], ks = p.cu_k[s];
        const int64_t jj = j - ks, off = (int64_t)(p.cu_k[s + 1] - ks) - (qe - qs);
        int64_t lo = qs, hi = qe;
        switch (p.mode[s]) {
          case FMASK_VL_CAUSAL: lo = qs + jj; break;
          case FMASK_VL_CAUSAL_BOTTOM_RIGHT: lo = qs + jj - off; break;
          case FMASK_VL_BAND:
            lo = qs + jj - p.next - off;
            hi = qs + jj + p.pre - off + 1;
            break;
          case FMASK_VL_PREFIX:
            if (jj >= p.prefix[s]) lo = qs + jj - off;
            break;
          default: break;  // FMASK_VL_FULL
        }
        vlo = lo > qs ? lo : qs;
        vhi = hi < qe ? hi : qe;
        break;
      }
      case FMASK_TREE: {  // prefix columns: causal; draft column c: its subtree rows
        vlo = j;
        if (j >= p.tree_prefix) vhi = (int64_t)p.tree_prefix + p.tree_hi[j - p.tree_prefix] + 1;
        break;
      }
      default:
        vlo = 0;
        vhi = 0;
        break;
    }
    store_visible_range(iv, p.skv, j, vlo, vhi, p.sq);
  }
}

// Canonicalise caller-supplied (UTS, UTE, LTS, LTE): clip to [0, sq], drop
// empty runs, order, merge overlapping or abutting runs.
__global__ void k_raw_intervals(const int32_t* raw, int32_t nmask, int32_t sq, int32_t skv,
                                int32_t* iv) {
  int64_t total = (int64_t)nmask * skv;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    int64_t m = t / skv, j = t % skv;
    const int32_t* r = raw + m * 4 * (int64_t)skv;
    int32_t a0 = min(max(r[j], 0), sq), b0 = min(max(r[skv + j], 0), sq);
    int32_t a1 = min(max(r[2 * (int64_t)skv + j], 0), sq), b1 = min(max(r[3 * (int64_t)skv + j], 0), sq);
    bool e0 = a0 >= b0, e1 = a1 >= b1;
    int32_t n = 0, s0 = 0, t0 = 0, s1 = 0, t1 = 0;
    if (!e0 && !e1) {
      if (a1 < a0) { int32_t x = a0; a0 = a1; a1 = x; x = b0; b0 = b1; b1 = x; }
      if (a1 <= b0) { n = 1; s0 = a0; t0 = max(b0, b1); }
      else { n = 2; s0 = a0; t0 = b0; s1 = a1; t1 = b1; }
    } else if (!e0) { n = 1; s0 = a0; t0 = b0; }
    else if (!e1) { n = 1; s0 = a1; t0 = b1; }
    int32_t uts = 0, ute = 0, lts = sq, lte = sq;
    if (n == 1) {
      if (s0 == 0) ute = t0; else { lts = s0; lte = t0; }
    } else if (n == 2) {
      uts = s0; ute = t0; lts = s1; lte = t1;
    }
    int32_t* o = iv + m * 4 * (int64_t)skv;
    o[j] = uts;
    o[skv + j] = ute;
    o[2 * (int64_t)skv + j] = lts;
    o[3 * (int64_t)skv + j] = lte;
  }
}

// Last descendant of every draft node (parent[t] < t, so a subtree that is a
// contiguous range is [c, hi[c]]).  One workgroup.
__global__ void k_tree_hi(const int32_t* parent, int32_t n, int32_t* hi) {
  for (int t = threadIdx.x; t < n; t += blockDim.x) hi[t] = t;
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    int a = parent[t];
    while (a >= 0) {
      atomicMax(&hi[a], t);
      a = parent[a];
    }
  }
}

// ------------------------------------------------------------------ dense
// The masked rows of one column over a range of rows, as at most two maximal
// runs [s0, e0), [s1, e1) and their number n (capped at 3: more than two).
struct Runs {
  int32_t n, s0, e0, s1, e1;
};
static_assert(sizeof(Runs) == 20, "partial-run records are 20 bytes");

// a then b, where b's rows follow a's: a run of b that starts where a's last
// run ends continues it.
__device__ inline Runs join(Runs a, Runs b) {
  if (b.n == 0) return a;
  if (a.n == 0) return b;
  if (a.n >= 3 || b.n >= 3) return Runs{3, 0, 0, 0, 0};
  const int32_t last_e = a.n == 1 ? a.e0 : a.e1;
  if (last_e == b.s0) {  // the two runs meet
    if (a.n == 1) return Runs{b.n, a.s0, b.e0, b.s1, b.e1};
    if (b.n == 1) return Runs{2, a.s0, a.e0, a.s1, b.e0};
    return Runs{3, 0, 0, 0, 0};
  }
  if (a.n + b.n > 2) return Runs{3, 0, 0, 0, 0};
  return Runs{2, a.s0, a.e0, b.s0, b.e0};
}

__device__ inline int32_t ctz64(uint64_t w) { return w ? __builtin_ctzll(w) : 64; }

// Runs of the set bits of w (bit r = row base + r masked).
__device__ inline Runs runs_of(uint64_t w, int32_t base) {
  Runs r{0, 0, 0, 0, 0};
  const int32_t starts = __popcll(w & ~(w << 1));
  if (starts == 0) return r;
  if (starts > 2) return Runs{3, 0, 0, 0, 0};
  const int32_t s0 = ctz64(w);
  const int32_t e0 = s0 + ctz64(~(w >> s0));
  r.n = starts;
  r.s0 = base + s0;
  r.e0 = base + e0;
  if (starts == 2) {
    const uint64_t rest = w & ~((e0 >= 64 ? ~0ull : (1ull << e0) - 1ull));
    const int32_t s1 = ctz64(rest);
    r.s1 = base + s1;
    r.e1 = base + s1 + ctz64(~(rest >> s1));
  }
  return r;
}

typedef int32_t dense_x4 __attribute__((ext_vector_type(4)));
__device__ dense_x4 dense_load16(rsrc_t rsrc, int voffset, int soffset, int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ uint32_t write_lane(uint32_t value, uint32_t lane, uint32_t old) __asm("llvm.amdgcn.writelane.i32");

// One workgroup (16 waves) per (mask, column strip); lane = column in the
// end.  Wave w walks its own contiguous share of the rows 64 at a time,
// turning each 64-row chunk of its columns into one bit word per column and
// that word into runs; the 16 shares are then joined in row order through LDS.
// A mask with a column of more than two runs raises *bad.
//   ROWS (Skv a multiple of 16): strips of 128 columns, so that a wave reads
//     whole 128-byte lines (with 64-column strips the two halves of a line
//     went to workgroups on different XCDs and every line was fetched twice).
//     Lane r reads the 128 bytes of chunk row r with eight 16-byte loads, and
//     one ballot per column turns the 64 rows' bytes into that column's word,
//     which v_writelane drops into lane (column % 64) of the word pair of
//     its half of the strip; a lane ends up with two columns.
//   otherwise: strips of 64 columns, lane = column throughout, one byte per
//     lane and row (a wave reads 64 consecutive bytes of a row).
constexpr int kDenseWaves = 16;

// Canonical intervals of a column from its runs (more than two: flag the mask).
__device__ inline void dense_store(const Runs& acc, int32_t sq, int32_t skv, int64_t m, int32_t j, int32_t* iv,
                                   int32_t* bad) {
  int32_t uts = 0, ute = 0, lts = sq, lte = sq;
  if (acc.n == 1) {
    if (acc.s0 == 0) ute = acc.e0; else { lts = acc.s0; lte = acc.e0; }
  } else if (acc.n == 2) {
    uts = acc.s0; ute = acc.e0; lts = acc.s1; lte = acc.e1;
  } else if (acc.n > 2) {
    atomicOr(bad, 1);
  }
  int32_t* o = iv + m * 4 * (int64_t)skv;
  o[j] = uts;
  o[skv + j] = ute;
  o[2 * (int64_t)skv + j] = lts;
  o[3 * (int64_t)skv + j] = lte;
}

// Workgroup (m, strip, g) covers rows [g * grows, (g + 1) * grows) of the
// strip; with one group it writes the intervals, else its joined runs go to
// ws[m][g][column] for k_dense_join.
template <bool ROWS>
__global__ void __launch_bounds__(1024) k_dense_intervals(const uint8_t* dense, int32_t sq, int32_t skv,
                                                          int32_t nstrip, int32_t ngroup, int32_t grows,
                                                          Runs* ws, int32_t* iv, int32_t* bad) {
  constexpr int SW = dense_strip(ROWS);  // columns per strip
  constexpr int NC = SW / 64;            // columns per lane
  __shared__ Runs part[kDenseWaves][SW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t g = blockIdx.x % ngroup;
  const int64_t m = blockIdx.x / ((int64_t)ngroup * nstrip);
  const int32_t c0 = (int32_t)((blockIdx.x / ngroup) % nstrip) * SW, j = c0 + lane;
  const int32_t g0 = g * grows, g1 = min(sq, g0 + grows);
  const int32_t share = (((grows + kDenseWaves - 1) / kDenseWaves) + 63) & ~63;
  const int32_t r0 = g0 + wave * share, r1 = min(g1, r0 + share);
  Runs acc[NC];
#pragma unroll
  for (int h = 0; h < NC; ++h) acc[h] = Runs{0, 0, 0, 0, 0};
  if (ROWS) {
    // rows [base, base + rows) of mask m; lanes past the chunk and bytes past
    // the mask read zeros, columns past skv (whose bytes are the next row's,
    // or zeros past the mask) are never written out
    auto load = [&](int32_t base, dense_x4* d) {  // (an empty range past the share: zeros)
      const rsrc_t r = make_rsrc(dense + ((size_t)m * sq + base) * skv, (int64_t)max(0, min(64, r1 - base)) * skv);
#pragma unroll
      for (int k = 0; k < SW / 16; ++k) d[k] = dense_load16(r, lane * skv + c0 + 16 * k, 0, 0);
    };
    dense_x4 d[SW / 16], dn[SW / 16];
    load(r0, d);
    for (int32_t base = r0; base < r1; base += 64) {
      const int32_t rows = min(64, r1 - base);
      load(base + 64, dn);  // the next chunk's bytes fly during this one
      const int32_t past = lane >= rows ? 0x01010101 : 0;  // rows past the chunk: visible (not masked)
#pragma unroll
      for (int k = 0; k < SW / 16; ++k) d[k] |= past;
      uint32_t wlo[NC], whi[NC];  // masked rows of columns c0 + 64 h + lane
#pragma unroll
      for (int h = 0; h < NC; ++h) wlo[h] = whi[h] = 0;
#pragma unroll
      for (int col = 0; col < SW; ++col) {
        const uint32_t byte = ((uint32_t)d[col >> 4][(col >> 2) & 3] >> (8 * (col & 3))) & 0xffu;
        const uint64_t vis = __ballot(byte != 0u);
        wlo[col >> 6] = write_lane(~(uint32_t)vis, col & 63, wlo[col >> 6]);
        whi[col >> 6] = write_lane(~(uint32_t)(vis >> 32), col & 63, whi[col >> 6]);
      }
#pragma unroll
      for (int h = 0; h < NC; ++h) acc[h] = join(acc[h], runs_of(((uint64_t)whi[h] << 32) | wlo[h], base));
#pragma unroll
      for (int k = 0; k < SW / 16; ++k) d[k] = dn[k];
    }
  } else if (j < skv) {
    const uint8_t* col = dense + (size_t)m * sq * skv + j;
    for (int32_t base = r0; base < r1; base += 64) {
      const int32_t rows = min(64, r1 - base);
      uint64_t w = 0;
      if (rows == 64) {
#pragma unroll 16
        for (int r = 0; r < 64; ++r) w |= (uint64_t)(col[(size_t)(base + r) * skv] == 0) << r;
      } else {
        for (int r = 0; r < rows; ++r) w |= (uint64_t)(col[(size_t)(base + r) * skv] == 0) << r;
      }
      acc[0] = join(acc[0], runs_of(w, base));
    }
  }
#pragma unroll
  for (int h = 0; h < NC; ++h) part[wave][64 * h + lane] = acc[h];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int h = 0; h < NC; ++h) {
    const int32_t jh = j + 64 * h;
    if (jh >= skv) break;
    Runs a = acc[h];
    for (int k = 1; k < kDenseWaves; ++k) a = join(a, part[k][64 * h + lane]);
    if (ngroup == 1) dense_store(a, sq, skv, m, jh, iv, bad);
    else ws[(m * ngroup + g) * skv + jh] = a;
  }
}

// The row groups of each (mask, column) joined in row order.
__global__ void k_dense_join(const Runs* ws, int64_t nmask, int32_t ngroup, int32_t sq, int32_t skv, int32_t* iv,
                             int32_t* bad) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < nmask * skv;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = t / skv;
    const int32_t j = (int32_t)(t % skv);
    Runs acc{0, 0, 0, 0, 0};
    for (int g = 0; g < ngroup; ++g) acc = join(acc, ws[(m * ngroup + g) * skv + j]);
    dense_store(acc, sq, skv, m, j, iv, bad);
  }
}

__global__ void k_zero_int(int32_t* x) { *x = 0; }

// ------------------------------------------------------------------ bitmap
__device__ inline uint64_t col_mask(int32_t skv, int bj) {
  int valid = skv - bj * kBlk;
  return valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
}

// Row word r of block (bi, bj) of mask m: bit c = vis(64 bi + r, 64 bj + c).
__device__ uint64_t source_word(const BitmapSrc& s, int m, int bi, int bj, int r) {
  int64_t i = (int64_t)bi * kBlk + r;
  if (i >= s.sq) return 0;
  uint64_t w = 0;
  if (s.kind == 0) {
    size_t b = ((size_t)m * s.nbq + bi) * s.nbk + bj;
    uint8_t st = s.state[b];
    if (st == FMASK_FULL) {
      w = ~0ull;
    } else if (st == FMASK_PARTIAL) {
      int64_t idx = s.index[b];
      if (idx >= 0 && idx < s.pool_n) w = s.bits[idx * kBlk + r];
    }
    if (s.force_diag) {
      int64_t c = i - (int64_t)bj * kBlk;
      if (c >= 0 && c < 64) w |= 1ull << c;
    }
  } else if (s.kind == 2) {
    // dense bytes of row i, columns 64 bj .. 64 bj + 63 (nonzero = visible)
    const uint8_t* row = s.dense + ((size_t)m * s.sq + i) * s.skv + (size_t)bj * kBlk;
    const int valid = min(64, s.skv - bj * kBlk);
    if (s.dense_vec && valid == 64) {
      // four 16-byte loads; bit 7 of ((b & 0x7f) + 0x7f) | b is set iff byte b
      // is nonzero (no carry leaves the byte), then those bits are gathered
      const uint4* row16 = (const uint4*)row;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = row16[q];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t t = ((((d[k] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | d[k]) & 0x80808080u) >> 7;
          const uint32_t nib = (t & 1u) | ((t >> 7) & 2u) | ((t >> 14) & 4u) | ((t >> 21) & 8u);
          w |= (uint64_t)nib << (16 * q + 4 * k);
        }
      }
    } else {
      for (int c = 0; c < valid; ++c) w |= (uint64_t)(row[c] != 0) << c;
    }
  } else {
    int64_t P = s.tree_prefix;
    int64_t base = (int64_t)bj * kBlk;
    if (i < P) {  // causal prefix row: columns j <= i
      int64_t c = i - base;
      w = c >= 63 ? ~0ull : (c >= 0 ? ((2ull << c) - 1ull) : 0ull);
    } else {      // draft row: whole prefix, then ancestors and itself
      int64_t pc = P - base;
      w = pc >= 64 ? ~0ull : (pc > 0 ? ((1ull << pc) - 1ull) : 0ull);
      int a = (int)(i - P);
      while (a >= 0) {
        int64_t c = P + a - base;
        if (c >= 0 && c < 64) w |= 1ull << c;
        a = s.parent[a];
      }
    }
  }
  return w & col_mask(s.skv, bj);
}

// One wave per block: exact state from the 64 row words.
__global__ void __launch_bounds__(256) k_bitmap_state(BitmapSrc s, uint8_t* state) {
  int64_t nblocks = (int64_t)s.nmask * s.nbq * s.nbk;
  int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int r = threadIdx.x & 63;
  if (blk >= nblocks) return;  // whole wave leaves together
  int bj = (int)(blk % s.nbk);
  int bi = (int)((blk / s.nbk) % s.nbq);
  int m = (int)(blk / ((int64_t)s.nbk * s.nbq));
  uint64_t w = source_word(s, m, bi, bj, r);
  bool row_valid = (int64_t)bi * kBlk + r < s.sq;
  bool full = !row_valid || w == col_mask(s.skv, bj);
  bool any = __any(w != 0);
  bool all = __all(full);
  if (r == 0) state[blk] = any ? (all ? FMASK_FULL : FMASK_PARTIAL) : FMASK_SKIP;
}

// Caller bitmaps (kind 0): one wave per 64 consecutive blocks, lane = block.
// A block whose input state is FULL stays FULL (its words are all visible, on
// ragged edges too) and one that is neither FULL nor PARTIAL stays SKIP (its
// words are zero), unless force_diag puts diagonal cells into it; the rest
// (PARTIAL input, diagonal blocks) are decided exactly from their 64 row words
// by the whole wave, one block at a time.  Same states as k_bitmap_state, with
// one wave per 64 blocks instead of one per block.
__global__ void __launch_bounds__(256) k_bitmap_state_lanes(BitmapSrc s, uint8_t* state) {
  const int64_t nblocks = (int64_t)s.nmask * s.nbq * s.nbk;
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int lane = threadIdx.x & 63;
  if (b0 >= nblocks) return;  // whole wave leaves together
  const int64_t b = b0 + lane;
  bool exact = false;
  if (b < nblocks) {
    const int bj = (int)(b % s.nbk);
    const int bi = (int)((b / s.nbk) % s.nbq);
    const uint8_t st = s.state[b];
    if (st == FMASK_FULL) state[b] = FMASK_FULL;
    else if (st == FMASK_PARTIAL || (s.force_diag && bi == bj)) exact = true;
    else state[b] = FMASK_SKIP;
  }
  uint64_t todo = __ballot(exact);
  while (todo) {
    const int64_t blk = b0 + __builtin_ctzll(todo);
    todo &= todo - 1;
    const int bj = (int)(blk % s.nbk);
    const int bi = (int)((blk / s.nbk) % s.nbq);
    const int m = (int)(blk / ((int64_t)s.nbk * s.nbq));
    const uint64_t w = source_word(s, m, bi, bj, lane);
    const bool row_valid = (int64_t)bi * kBlk + lane < s.sq;
    const bool full = !row_valid || w == col_mask(s.skv, bj);
    const bool any = __any(w != 0);
    const bool all = __all(full);
    if (lane == 0) state[blk] = any ? (all ? FMASK_FULL : FMASK_PARTIAL) : FMASK_SKIP;
  }
}

// One wave per block row: row-local rank of every PARTIAL block, and the count.
__global__ void __launch_bounds__(256) k_bitmap_row_rank(const uint8_t* state, int32_t rows,
                                                         int32_t nbk, int32_t* index,
                                                         int32_t* row_count) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  int lane = threadIdx.x & 63;
  if (row >= rows) return;
  int running = 0;
  for (int base = 0; base < nbk; base += 64) {
    int bj = base + lane;
    bool part = bj < nbk && state[(int64_t)row * nbk + bj] == FMASK_PARTIAL;
    uint64_t bal = __ballot(part);
    int rank = running + __popcll(bal & ((1ull << lane) - 1ull));
    if (bj < nbk) index[(int64_t)row * nbk + bj] = part ? rank : -1;
    running += __popcll(bal);
  }
  if (lane == 0) row_count[row] = running;
}

// Exclusive scan of n counts (one workgroup of 1024 threads), total to *total.
__global__ void __launch_bounds__(1024) k_exclusive_scan(const int32_t* in, int32_t n, int32_t* out,
                                                         int32_t* total) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    int i = base + threadIdx.x;
    int32_t x = i < n ? in[i] : 0;
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int32_t y = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += y;
      __syncthreads();
    }
    int32_t incl = buf[threadIdx.x];
    int32_t c = carry;
    if (i < n) out[i] = c + incl - x;
    __syncthreads();
    if (threadIdx.x == 1023) carry = c + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

// One wave per block: final pool index, and the 64 words of PARTIAL blocks.
__global__ void __launch_bounds__(256) k_bitmap_words(BitmapSrc s, BitmapOut o) {
  int64_t nblocks = (int64_t)s.nmask * s.nbq * s.nbk;
  int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  int r = threadIdx.x & 63;
  if (blk >= nblocks) return;
  int32_t local = o.index[blk];
  if (local < 0) return;  // uniform over the wave
  int bj = (int)(blk % s.nbk);
  int64_t row = blk / s.nbk;
  int bi = (int)(row % s.nbq);
  int m = (int)(row / s.nbq);
  int64_t g = (int64_t)o.row_offset[row] + local;
  __builtin_amdgcn_wave_barrier();
  if (r == 0) o.index[blk] = (int32_t)g;
  if (g < o.cap) o.bits[g * kBlk + r] = source_word(s, m, bi, bj, r);
}

// Caller bitmaps: one wave per 64 consecutive blocks; the wave writes the
// pool words of its PARTIAL blocks one block at a time (lane = row), as
// k_bitmap_words does with one wave per block.
__global__ void __launch_bounds__(256) k_bitmap_words_lanes(BitmapSrc s, BitmapOut o) {
  const int64_t nblocks = (int64_t)s.nmask * s.nbq * s.nbk;
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  const int lane = threadIdx.x & 63;
  if (b0 >= nblocks) return;  // whole wave leaves together
  const int32_t local = b0 + lane < nblocks ? o.index[b0 + lane] : -1;
  uint64_t todo = __ballot(local >= 0);
  while (todo) {
    const int src = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int64_t blk = b0 + src;
    const int bj = (int)(blk % s.nbk);
    const int64_t row = blk / s.nbk;
    const int bi = (int)(row % s.nbq);
    const int m = (int)(row / s.nbq);
    const int64_t g = (int64_t)o.row_offset[row] + __shfl(local, src);
    if (lane == 0) o.index[blk] = (int32_t)g;  // every lane read its index before the loop
    if (g < o.cap) o.bits[g * kBlk + lane] = source_word(s, m, bi, bj, lane);
  }
}

// ------------------------------------------------------------------ selected
// One wave per (batch, query): keep the valid first occurrences, rank them.
__global__ void __launch_bounds__(256) k_selected_canon(const int32_t* sel, int32_t nb, int32_t sq,
                                                        int32_t n, int32_t nblk, int32_t* list,
                                                        int32_t* count) {
  __shared__ int32_t vals[4][64];
  __shared__ int32_t keep[4][64];
  int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t q = (int64_t)blockIdx.x * 4 + w;
  bool live = q < (int64_t)nb * sq;
  int32_t x = (live && lane < n) ? sel[q * n + lane] : -1;
  bool valid = live && lane < n && x >= 0 && x < nblk;
  vals[w][lane] = valid ? x : -1;
  __syncthreads();
  bool first = valid;
  for (int e = 0; e < lane && first; ++e) first = vals[w][e] != x;
  keep[w][lane] = first;
  __syncthreads();
  if (!live) return;
  int rank = 0, total = 0;
  for (int e = 0; e < n; ++e) {
    if (keep[w][e]) {
      ++total;
      rank += vals[w][e] < x;
    }
  }
  if (first) list[q * n + rank] = x;
  if (lane < n && lane >= total) list[q * n + lane] = -1;
  if (lane == 0) count[q] = total;
}

inline int grid_for(int64_t n, int per_block, int cap = 65535 * 16) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

}  // namespace

hipError_t launch_encode_family_intervals(const SegParams& p, int32_t* iv, hipStream_t s) {
  if (p.skv <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_family_intervals, dim3(grid_for(p.skv, 256)), dim3(256), 0, s, p, iv);
  return hipGetLastError();
}

hipError_t launch_encode_raw_intervals(const int32_t* raw, int32_t nmask, int32_t sq, int32_t skv,
                                       int32_t* iv, hipStream_t s) {
  int64_t total = (int64_t)nmask * skv;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_raw_intervals, dim3(grid_for(total, 256)), dim3(256), 0, s, raw, nmask, sq,
                     skv, iv);
  return hipGetLastError();
}

hipError_t launch_tree_hi(const int32_t* parent, int32_t n, int32_t* hi, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_tree_hi, dim3(1), dim3(1024), 0, s, parent, n, hi);
  return hipGetLastError();
}

hipError_t launch_encode_bitmap(const BitmapSrc& src, const BitmapOut& out, hipStream_t s) {
  int64_t nblocks = (int64_t)src.nmask * src.nbq * src.nbk;
  int32_t rows = src.nmask * src.nbq;
  if (nblocks <= 0) return hipSuccess;
  int g4 = (int)((nblocks + 3) / 4);
  const int g256 = (int)((nblocks + 255) / 256);
  if (src.kind == 0) hipLaunchKernelGGL(k_bitmap_state_lanes, dim3(g256), dim3(256), 0, s, src, out.state);
  else hipLaunchKernelGGL(k_bitmap_state, dim3(g4), dim3(256), 0, s, src, out.state);
  hipLaunchKernelGGL(k_bitmap_row_rank, dim3((rows + 3) / 4), dim3(256), 0, s, out.state, rows,
                     src.nbk, out.index, out.row_count);
  hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(1024), 0, s, out.row_count, rows,
                     out.row_offset, out.pool_count);
  if (src.kind == 0) hipLaunchKernelGGL(k_bitmap_words_lanes, dim3(g256), dim3(256), 0, s, src, out);
  else hipLaunchKernelGGL(k_bitmap_words, dim3(g4), dim3(256), 0, s, src, out);
  return hipGetLastError();
}

hipError_t launch_zero_int(int32_t* x, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(1), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_encode_dense_intervals(const uint8_t* dense, int32_t nmask, int32_t sq, int32_t skv,
                                         void* ws, int32_t* iv, int32_t* bad, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_int, dim3(1), dim3(1), 0, s, bad);
  const bool rows = skv % 16 == 0 && (uintptr_t)dense % 16 == 0 && (int64_t)64 * skv < ((int64_t)1 << 31);
  const int32_t nstrip = (skv + dense_strip(rows) - 1) / dense_strip(rows);
  const int32_t ngroup = dense_groups(nmask, sq, skv);
  const int32_t grows = (int32_t)((((int64_t)sq + ngroup - 1) / ngroup + 63) / 64 * 64);
  const int64_t blocks = (int64_t)nmask * nstrip * ngroup;
  if (blocks <= 0) return hipGetLastError();
  // 16-byte row loads need 16-byte aligned rows; 64 rows must stay within the
  // 32-bit buffer offsets
  if (rows)
    hipLaunchKernelGGL(k_dense_intervals<true>, dim3((unsigned)blocks), dim3(1024), 0, s, dense, sq, skv,
                       nstrip, ngroup, grows, (Runs*)ws, iv, bad);
  else
    hipLaunchKernelGGL(k_dense_intervals<false>, dim3((unsigned)blocks), dim3(1024), 0, s, dense, sq, skv,
                       nstrip, ngroup, grows, (Runs*)ws, iv, bad);
  if (ngroup > 1)
    hipLaunchKernelGGL(k_dense_join, dim3(grid_for((int64_t)nmask * skv, 256)), dim3(256), 0, s, (const Runs*)ws,
                       (int64_t)nmask, ngroup, sq, skv, iv, bad);
  return hipGetLastError();
}

hipError_t launch_encode_selected(const int32_t* sel, int32_t nb, int32_t sq, int32_t n,
                                  int32_t nblk, int32_t* list, int32_t* count, hipStream_t s) {
  int64_t q = (int64_t)nb * sq;
  if (q <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_selected_canon, dim3((unsigned)((q + 3) / 4)), dim3(256), 0, s, sel, nb, sq,
                     n, nblk, list, count);
  return hipGetLastError();
}

}  // namespace fmask
