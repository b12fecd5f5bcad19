// libfmask C ABI: argument checking, buffer layout and kernel launches.
// Every host-detectable error is reported before anything is launched; the
// library never allocates, frees or synchronises (the no-allocation split form
// uses a fixed scratch array that is part of the library's code object).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "internal.h"

using namespace fmask;

namespace {

thread_local char g_err[512] = "";

fmask_status fail(fmask_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

fmask_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FMASK_OK;
  return fail(FMASK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxSeq = (int64_t)1 << 30;
constexpr int32_t kMaxTree = 4096;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Every buffer the library sizes stays below 2^44 bytes (far past any GPU's
// memory), so that the size arithmetic below never overflows.
constexpr int64_t kMaxBytes = (int64_t)1 << 44;

// Product of non-negative factors when it is at most lim, else -1; no partial
// product overflows (a zero factor gives 0 whatever the others are).
int64_t bounded_prod(std::initializer_list<int64_t> xs, int64_t lim) {
  for (int64_t x : xs)
    if (x == 0) return 0;
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x < 0 || r > lim / x) return -1;
    r *= x;
  }
  return r;
}
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

bool is_segment_family(int f) {
  return f == FMASK_DOCUMENT || f == FMASK_CAUSAL_DOCUMENT || f == FMASK_SHARED_QUESTION;
}

bool is_param_family(int f) {
  return f == FMASK_CAUSAL || f == FMASK_CAUSAL_BOTTOM_RIGHT || f == FMASK_BAND || f == FMASK_TREE ||
         f == FMASK_VARLEN || is_segment_family(f);
}

// Tree analysis on the host copy of the parent array: validity, and whether
// every subtree is a contiguous node range (then the interval form holds).
fmask_status tree_check(const fmask_mask_desc* d, bool* contiguous) {
  const int n = d->tree_n;
  std::vector<int> size(n, 0), hi(n, 0);
  for (int t = 0; t < n; ++t) {
    int p = d->tree_parent[t];
    if (p < -1 || p >= t) return fail(FMASK_ERR_INVALID, "tree_parent[%d] = %d is not in [-1, %d)", t, p, t);
  }
  for (int t = 0; t < n; ++t) {
    for (int a = t; a >= 0; a = d->tree_parent[a]) {
      size[a] += 1;
      hi[a] = std::max(hi[a], t);
    }
  }
  bool ok = true;
  for (int c = 0; c < n && ok; ++c) ok = size[c] == hi[c] - c + 1;
  *contiguous = ok;
  return FMASK_OK;
}

fmask_status check_family(const fmask_mask_desc* d, int* kind);

fmask_status check_desc(const fmask_mask_desc* d, int* kind) {
  if (!d) return fail(FMASK_ERR_INVALID, "null mask descriptor");
  if (d->sq < 0 || d->skv < 0 || d->sq > kMaxSeq || d->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "sq / skv out of range [0, 2^30]");
  if (d->batch < 1 || d->heads < 1) return fail(FMASK_ERR_INVALID, "batch and heads must be >= 1");
  const int64_t nmask = (int64_t)d->batch * d->heads;
  if (nmask > INT32_MAX) return fail(FMASK_ERR_UNSUPPORTED, "batch * heads: at most 2^31 - 1 masks");
  const fmask_status st = check_family(d, kind);
  if (st != FMASK_OK) return st;
  // storage of the encoding (the automatic dense form reserves both forms)
  const bool dense_auto = d->family == FMASK_DENSE && d->dense_form == 0;
  bool fits = true;
  if (*kind == FMASK_ENC_INTERVALS) fits = bounded_prod({nmask, d->skv, 16}, kMaxBytes) >= 0;
  if (*kind == FMASK_ENC_BITMAP || dense_auto)
    fits = fits && bounded_prod({nmask, ceil_div(d->sq, kBlk), ceil_div(d->skv, kBlk), kBlk * 8 + 8}, kMaxBytes) >= 0;
  if (*kind == FMASK_ENC_SELECTED) fits = bounded_prod({d->batch, d->sq, d->sel_n, 4}, kMaxBytes) >= 0;
  if (!fits) return fail(FMASK_ERR_UNSUPPORTED, "the encoding would exceed 2^44 bytes");
  return FMASK_OK;
}

// Family-specific checks of a descriptor; sets the kind it encodes to.
fmask_status check_family(const fmask_mask_desc* d, int* kind) {
  const int f = d->family;
  if (is_param_family(f) && (d->batch != 1 || d->heads != 1))
    return fail(FMASK_ERR_INVALID, "family %d describes one mask: batch = heads = 1", f);
  switch (f) {
    case FMASK_CAUSAL:
    case FMASK_CAUSAL_BOTTOM_RIGHT:
    case FMASK_BAND:
      *kind = FMASK_ENC_INTERVALS;
      return FMASK_OK;
    case FMASK_DOCUMENT:
    case FMASK_CAUSAL_DOCUMENT:
    case FMASK_SHARED_QUESTION: {
      if (d->sq != d->skv) return fail(FMASK_ERR_INVALID, "segment families need sq == skv");
      if (!d->cu_seg || d->n_seg < 1) return fail(FMASK_ERR_INVALID, "cu_seg missing or n_seg < 1");
      if (d->cu_seg[0] != 0) return fail(FMASK_ERR_INVALID, "cu_seg[0] must be 0");
      for (int s = 0; s < d->n_seg; ++s)
        if (d->cu_seg[s + 1] <= d->cu_seg[s])
          return fail(FMASK_ERR_INVALID, "cu_seg not strictly increasing at %d", s);
      if (d->cu_seg[d->n_seg] != d->sq) return fail(FMASK_ERR_INVALID, "cu_seg[n_seg] != sq");
      *kind = FMASK_ENC_INTERVALS;
      return FMASK_OK;
    }
    case FMASK_VARLEN: {
      if (!d->cu_seg || !d->cu_seg_k || !d->seg_mode || d->n_seg < 1)
        return fail(FMASK_ERR_INVALID, "varlen needs cu_seg, cu_seg_k, seg_mode and n_seg >= 1");
      if (d->n_seg > (1 << 24)) return fail(FMASK_ERR_INVALID, "too many segments");
      if (d->cu_seg[0] != 0 || d->cu_seg_k[0] != 0)
        return fail(FMASK_ERR_INVALID, "cu_seg[0] and cu_seg_k[0] must be 0");
      for (int s = 0; s < d->n_seg; ++s) {
        if (d->cu_seg[s + 1] < d->cu_seg[s] || d->cu_seg_k[s + 1] < d->cu_seg_k[s])
          return fail(FMASK_ERR_INVALID, "cumulative lengths decrease at segment %d", s);
        const int m = d->seg_mode[s];
        if (m < FMASK_VL_FULL || m > FMASK_VL_PREFIX)
          return fail(FMASK_ERR_INVALID, "seg_mode[%d] = %d is not a varlen mode", s, m);
        if (m == FMASK_VL_PREFIX && (!d->seg_prefix || d->seg_prefix[s] < 0))
          return fail(FMASK_ERR_INVALID, "seg_prefix[%d] missing or negative", s);
      }
      if (d->cu_seg[d->n_seg] != d->sq || d->cu_seg_k[d->n_seg] != d->skv)
        return fail(FMASK_ERR_INVALID, "cumulative lengths must end at sq and skv");
      *kind = FMASK_ENC_INTERVALS;
      return FMASK_OK;
    }
    case FMASK_TREE: {
      if (d->tree_n < 0 || d->tree_n > kMaxTree || d->tree_prefix < 0)
        return fail(FMASK_ERR_INVALID, "tree_n must be in [0, %d], tree_prefix >= 0", kMaxTree);
      if (d->sq != d->skv || d->sq != (int64_t)d->tree_prefix + d->tree_n)
        return fail(FMASK_ERR_INVALID, "tree needs sq == skv == tree_prefix + tree_n");
      if (d->tree_n > 0 && !d->tree_parent) return fail(FMASK_ERR_INVALID, "tree_parent missing");
      bool contiguous = true;
      fmask_status st = tree_check(d, &contiguous);
      if (st != FMASK_OK) return st;
      *kind = contiguous ? FMASK_ENC_INTERVALS : FMASK_ENC_BITMAP;
      return FMASK_OK;
    }
    case FMASK_BLOCK_BITMAP:
      if ((d->sq > 0 && d->skv > 0) && (!d->blk_state || !d->blk_index))
        return fail(FMASK_ERR_INVALID, "blk_state / blk_index missing");
      if (d->blk_pool_n < 0 || (d->blk_pool_n > 0 && !d->blk_bits))
        return fail(FMASK_ERR_INVALID, "blk_bits missing or blk_pool_n < 0");
      *kind = FMASK_ENC_BITMAP;
      return FMASK_OK;
    case FMASK_SELECTED_KEY:
      if (d->heads != 1) return fail(FMASK_ERR_INVALID, "selected-key lists are shared by all heads");
      if (d->sel_n < 1 || d->sel_n > FMASK_MAX_SEL_N)
        return fail(FMASK_ERR_INVALID, "sel_n must be in [1, %d]", FMASK_MAX_SEL_N);
      if (d->sel_cells < 1) return fail(FMASK_ERR_INVALID, "sel_cells must be >= 1");
      if (d->sq > 0 && !d->sel) return fail(FMASK_ERR_INVALID, "sel missing");
      *kind = FMASK_ENC_SELECTED;
      return FMASK_OK;
    case FMASK_INTERVALS:
      if (d->sq > 0 && d->skv > 0 && !d->raw_intervals)
        return fail(FMASK_ERR_INVALID, "raw_intervals missing");
      *kind = FMASK_ENC_INTERVALS;
      return FMASK_OK;
    case FMASK_DENSE:
      if (d->sq > 0 && d->skv > 0 && !d->dense) return fail(FMASK_ERR_INVALID, "dense mask missing");
      if (d->dense_form != 0 && d->dense_form != FMASK_ENC_INTERVALS && d->dense_form != FMASK_ENC_BITMAP)
        return fail(FMASK_ERR_INVALID, "dense_form must be 0, FMASK_ENC_INTERVALS or FMASK_ENC_BITMAP");
      if (bounded_prod({(int64_t)d->batch * d->heads, d->sq, d->skv}, (int64_t)1 << 40) < 0 ||
          (int64_t)d->batch * d->heads * ceil_div(d->skv, 64) > INT32_MAX)
        return fail(FMASK_ERR_UNSUPPORTED, "dense mask too large");
      // the interval form is tried first unless the bitmap form is asked for
      *kind = d->dense_form == FMASK_ENC_BITMAP ? FMASK_ENC_BITMAP : FMASK_ENC_INTERVALS;
      return FMASK_OK;
    default:
      return fail(FMASK_ERR_INVALID, "unknown mask family %d", f);
  }
}

struct EncLayout {
  int kind = 0;
  size_t total = 0;
  size_t iv = 0, cu = 0, parent = 0, tree_hi = 0, flag = 0, dws = 0;
  size_t bstate = 0, bindex = 0, bbits = 0, row_count = 0, row_offset = 0, pool_count = 0;
  size_t list = 0, count = 0;
  int64_t nbq = 0, nbk = 0, cap = 0;
};

EncLayout enc_layout(const fmask_mask_desc* d, int kind) {
  EncLayout L;
  L.kind = kind;
  Carve c;
  const int64_t nmask = (int64_t)d->batch * d->heads;
  // A dense mask of the automatic form may end up in either form: room for both.
  const bool dense_auto = d->family == FMASK_DENSE && d->dense_form == 0;
  if (d->family == FMASK_DENSE && kind == FMASK_ENC_INTERVALS) {
    L.flag = c.take(sizeof(int32_t));
    L.dws = c.take(std::max<size_t>(dense_ws_bytes(nmask, d->sq, d->skv), 16));
  }
  if (kind == FMASK_ENC_INTERVALS) {
    L.iv = c.take((size_t)nmask * 4 * d->skv * sizeof(int32_t));
    if (is_segment_family(d->family)) L.cu = c.take((size_t)(d->n_seg + 1) * sizeof(int32_t));
    // varlen: cu_q [n+1], cu_k [n+1], mode [n], prefix [n]
    if (d->family == FMASK_VARLEN) L.cu = c.take((size_t)(4 * (int64_t)d->n_seg + 2) * sizeof(int32_t));
    if (d->family == FMASK_TREE) {
      L.parent = c.take((size_t)std::max(1, d->tree_n) * sizeof(int32_t));
      L.tree_hi = c.take((size_t)std::max(1, d->tree_n) * sizeof(int32_t));
    }
  }
  if (kind == FMASK_ENC_BITMAP || dense_auto) {
    L.nbq = ceil_div(d->sq, kBlk);
    L.nbk = ceil_div(d->skv, kBlk);
    const int64_t nblocks = nmask * L.nbq * L.nbk;
    // Worst case: every block PARTIAL (the canonical pool is compact, this
    // only reserves room; no dense mask is ever written).
    L.cap = nblocks;
    L.bstate = c.take((size_t)nblocks);
    L.bindex = c.take((size_t)nblocks * sizeof(int32_t));
    L.bbits = c.take((size_t)L.cap * kBlk * sizeof(uint64_t));
    L.row_count = c.take((size_t)std::max<int64_t>(1, nmask * L.nbq) * sizeof(int32_t));
    L.row_offset = c.take((size_t)std::max<int64_t>(1, nmask * L.nbq) * sizeof(int32_t));
    L.pool_count = c.take(sizeof(int32_t));
    if (d->family == FMASK_TREE) L.parent = c.take((size_t)std::max(1, d->tree_n) * sizeof(int32_t));
  } else if (kind == FMASK_ENC_SELECTED) {
    L.list = c.take((size_t)d->batch * d->sq * d->sel_n * sizeof(int32_t));
    L.count = c.take((size_t)d->batch * d->sq * sizeof(int32_t));
  }
  L.total = std::max<size_t>(c.off, kAlign);
  return L;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

struct TileLayout {
  size_t state = 0, list = 0, count = 0, order = 0, total = 0;
  int64_t nqt = 0, nkt = 0, rows = 0;
};

fmask_status check_tiles_args(const fmask_encoded* e, int32_t bm, int32_t bn) {
  if (!e) return fail(FMASK_ERR_INVALID, "null encoding");
  if (e->kind != FMASK_ENC_INTERVALS && e->kind != FMASK_ENC_BITMAP)
    return fail(FMASK_ERR_INVALID, "tile tables exist for the INTERVALS and BITMAP kinds only");
  if (bm < 16 || bm > 256 || bn < 16 || bn > 256 || bm % 16 || bn % 16)
    return fail(FMASK_ERR_INVALID, "bm, bn must be multiples of 16 in [16, 256]");
  if (e->kind == FMASK_ENC_BITMAP && (bm % kBlk || bn % kBlk))
    return fail(FMASK_ERR_INVALID, "BITMAP tiles must be multiples of 64");
  if (e->batch < 1 || e->heads < 1 || e->sq < 0 || e->skv < 0 || e->sq > kMaxSeq || e->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "malformed encoding");
  const int64_t rows = bounded_prod({(int64_t)e->batch * e->heads, ceil_div(e->sq, bm)}, INT32_MAX);
  if (rows < 0 || bounded_prod({rows, ceil_div(e->skv, bn)}, (int64_t)1 << 40) < 0)
    return fail(FMASK_ERR_UNSUPPORTED, "tile table too large");
  return FMASK_OK;
}

// The mask data the interval and bitmap kernels index: present, and for the
// bitmap the block grid that sq and skv imply (a hand-filled descriptor with
// another grid would send the kernels outside the block arrays).
fmask_status check_mask_data(const fmask_encoded* e) {
  if (e->kind == FMASK_ENC_INTERVALS) {
    if (e->skv > 0 && !e->intervals) return fail(FMASK_ERR_INVALID, "null interval array");
  } else if (e->kind == FMASK_ENC_BITMAP) {
    if (e->blk != kBlk || e->nbq != ceil_div(e->sq, kBlk) || e->nbk != ceil_div(e->skv, kBlk))
      return fail(FMASK_ERR_INVALID, "bitmap block grid does not match sq / skv");
    if (e->nbq * e->nbk > 0 && (!e->blk_state || !e->blk_index || !e->blk_bits))
      return fail(FMASK_ERR_INVALID, "null bitmap array");
  }
  return FMASK_OK;
}

// Tensor pointers are required when their tensor holds an element: Q and O
// (and the backward's dO, dQ, LSE) for sq > 0, K and V (dK, dV) for skv > 0.
// A zero-length sequence may come with null pointers, as empty device
// tensors do.
bool present(int64_t extent, std::initializer_list<const void*> ptrs) {
  if (extent == 0) return true;
  for (const void* x : ptrs)
    if (!x) return false;
  return true;
}

TileLayout tile_layout(const fmask_encoded* e, int32_t bm, int32_t bn) {
  TileLayout T;
  Carve c;
  T.nqt = ceil_div(e->sq, bm);
  T.nkt = ceil_div(e->skv, bn);
  T.rows = (int64_t)e->batch * e->heads * T.nqt;
  T.state = c.take((size_t)T.rows * T.nkt);
  T.list = c.take((size_t)T.rows * T.nkt * sizeof(int32_t));
  T.count = c.take((size_t)T.rows * sizeof(int32_t));
  T.order = c.take((size_t)T.rows * sizeof(int32_t));
  T.total = std::max<size_t>(c.off, kAlign);
  return T;
}

// Tile shapes with a kernel: bf16 intervals 256x64, 128x64 and 64x64; bf16
// bitmap 128x64 and 64x64; fp32 64x64.
bool tile_supported(int32_t dtype, int32_t kind, int32_t bm, int32_t bn) {
  if (bn != 64) return false;
  if (dtype == FMASK_F32) return bm == 64;
  if (kind == FMASK_ENC_INTERVALS) return bm == 256 || bm == 128 || bm == 64;
  return bm == 64 || bm == 128;
}

void preferred(int32_t dtype, int32_t d, int32_t kind, int32_t* bm, int32_t* bn) {
  (void)d;
  *bn = 64;
  if (dtype == FMASK_F32) *bm = 64;
  else *bm = 128;
}

}  // namespace

// Checks and parameters of the selected-key kernels (shared by the one-pass
// and the split forms).
fmask_status selected_params(const fmask_attn_args* a, const void* q, const void* k, const void* v,
                             void* o, float* lse, const fmask_encoded* enc, SelAttnParams* p) {
  const int32_t group = a->hq / a->hkv;
  if (a->dtype != FMASK_BF16 || (a->d != 256 && a->d != 128) || enc->blk != 32 ||
      !selected_group_supported(group))
    return fail(FMASK_ERR_UNSUPPORTED, "selected-key kernel: bf16, d in {128, 256}, 32-cell blocks, "
                                       "hq/hkv in {1,2,4,8,12,16}");
  if (enc->heads != 1) return fail(FMASK_ERR_INVALID, "selected-key lists are shared by all heads");
  p->q = q; p->k = k; p->v = v; p->o = o; p->lse = lse;
  memcpy(p->qs, a->q_stride, sizeof(p->qs));
  memcpy(p->ks, a->k_stride, sizeof(p->ks));
  memcpy(p->vs, a->v_stride, sizeof(p->vs));
  memcpy(p->os, a->o_stride, sizeof(p->os));
  p->b = a->b; p->hq = a->hq; p->hkv = a->hkv; p->group = group;
  p->sq = (int32_t)a->sq; p->skv = (int32_t)a->skv; p->scale = a->scale;
  p->list = enc->sel_list; p->count = enc->sel_count;
  p->n = enc->sel_n; p->cells = enc->blk; p->mb = enc->batch;
  if (bounded_prod({(int64_t)a->hkv * a->b, a->sq, 16}, INT32_MAX) < 0)
    return fail(FMASK_ERR_UNSUPPORTED, "grid too large");
  return FMASK_OK;
}

// Splits per list for the split form: enough workgroups to cover the chip
// twice (256 CUs), at least 4 entries (one per wave) per split.
int32_t auto_splits(const fmask_attn_args* a, int32_t sel_n) {
  const int64_t items = (int64_t)a->hkv * a->b * a->sq;
  if (items <= 0) return 1;
  int64_t sp = (2 * 256 + items - 1) / items;
  const int64_t cap = std::max<int64_t>(1, (sel_n + 3) / 4);
  return (int32_t)std::min<int64_t>(std::max<int64_t>(sp, 1), cap);
}

extern "C" {

const char* fmask_status_str(fmask_status s) {
  switch (s) {
    case FMASK_OK: return "ok";
    case FMASK_ERR_INVALID: return "invalid argument";
    case FMASK_ERR_UNSUPPORTED: return "unsupported combination";
    case FMASK_ERR_CAPACITY: return "buffer too small";
    case FMASK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fmask_last_error(void) { return g_err; }

fmask_status fmask_preferred_tile(int32_t dtype, int32_t d, int32_t kind, int32_t* bm, int32_t* bn) {
  if (!bm || !bn) return fail(FMASK_ERR_INVALID, "null output pointer");
  if (kind != FMASK_ENC_INTERVALS && kind != FMASK_ENC_BITMAP)
    return fail(FMASK_ERR_INVALID, "tiles exist for the INTERVALS and BITMAP kinds only");
  if ((dtype != FMASK_BF16 && dtype != FMASK_F32) || (d != 64 && d != 128))
    return fail(FMASK_ERR_UNSUPPORTED, "no tile kernel for dtype %d, d %d", dtype, d);
  preferred(dtype, d, kind, bm, bn);
  return FMASK_OK;
}

size_t fmask_encode_bytes(const fmask_mask_desc* desc) {
  int kind = 0;
  if (check_desc(desc, &kind) != FMASK_OK) return 0;
  return enc_layout(desc, kind).total;
}

fmask_status fmask_encode(const fmask_mask_desc* desc, void* out, size_t out_bytes, fmask_encoded* enc,
                          void* stream) {
  g_err[0] = 0;
  int kind = 0;
  fmask_status st = check_desc(desc, &kind);
  if (st != FMASK_OK) return st;
  if (!enc) return fail(FMASK_ERR_INVALID, "null fmask_encoded");
  if (!out || ((uintptr_t)out % kAlign)) return fail(FMASK_ERR_INVALID, "out must be 256-byte aligned");
  const EncLayout L = enc_layout(desc, kind);
  if (out_bytes < L.total)
    return fail(FMASK_ERR_CAPACITY, "out has %zu bytes, %zu needed", out_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  const int f = desc->family;
  const int32_t sq = (int32_t)desc->sq, skv = (int32_t)desc->skv;
  const int32_t nmask = (int32_t)((int64_t)desc->batch * desc->heads);  // <= 2^31 - 1 (check_desc)

  memset(enc, 0, sizeof(*enc));
  enc->kind = kind;
  enc->batch = desc->batch;
  enc->heads = desc->heads;
  enc->sq = desc->sq;
  enc->skv = desc->skv;

  hipError_t e = hipSuccess;
  if (kind == FMASK_ENC_INTERVALS && f == FMASK_DENSE) {
    int32_t* iv = at<int32_t>(out, L.iv);
    int32_t* bad = at<int32_t>(out, L.flag);
    enc->intervals = iv;
    e = launch_encode_dense_intervals(desc->dense, nmask, sq, skv, at<char>(out, L.dws), iv, bad, s);
    if (e != hipSuccess) return hip_status(e, "dense encode kernel");
    int32_t hbad = 0;  // the one synchronising read: which form holds the mask
    e = hipMemcpyAsync(&hbad, bad, sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e, "read dense flag");
    if (!hbad) return FMASK_OK;
    if (desc->dense_form == FMASK_ENC_INTERVALS)
      return fail(FMASK_ERR_INVALID, "a column of the dense mask has more than two masked runs");
    kind = FMASK_ENC_BITMAP;  // automatic form: fall back to the bitmap encoding
    enc->kind = kind;
    enc->intervals = nullptr;
  }
  if (kind == FMASK_ENC_INTERVALS) {
    int32_t* iv = at<int32_t>(out, L.iv);
    enc->intervals = iv;
    if (f == FMASK_INTERVALS) {
      e = launch_encode_raw_intervals(desc->raw_intervals, nmask, sq, skv, iv, s);
    } else {
      SegParams p{};
      p.family = f;
      p.sq = sq;
      p.skv = skv;
      int64_t lim = (int64_t)sq + skv + 1;
      p.pre = std::min(std::max(desc->pre_tokens, -lim), lim);
      p.next = std::min(std::max(desc->next_tokens, -lim), lim);
      if (is_segment_family(f)) {
        p.n_seg = desc->n_seg;
        if (desc->n_seg <= kSegInline) {  // small: in the kernel's arguments
          memcpy(p.cu_inline, desc->cu_seg, (size_t)(desc->n_seg + 1) * sizeof(int32_t));
        } else {
          int32_t* cu = at<int32_t>(out, L.cu);
          e = hipMemcpyAsync(cu, desc->cu_seg, (size_t)(desc->n_seg + 1) * sizeof(int32_t),
                             hipMemcpyHostToDevice, s);
          if (e != hipSuccess) return hip_status(e, "copy cu_seg");
          p.cu = cu;
        }
      }
      if (f == FMASK_VARLEN) {
        const int n = desc->n_seg;
        int32_t* cu = at<int32_t>(out, L.cu);
        int32_t* cuk = cu + (n + 1);
        int32_t* md = cuk + (n + 1);
        int32_t* pf = md + n;
        e = hipMemcpyAsync(cu, desc->cu_seg, (size_t)(n + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
          e = hipMemcpyAsync(cuk, desc->cu_seg_k, (size_t)(n + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
          e = hipMemcpyAsync(md, desc->seg_mode, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e == hipSuccess && desc->seg_prefix)
          e = hipMemcpyAsync(pf, desc->seg_prefix, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, "copy varlen segments");
        p.cu = cu;
        p.cu_k = cuk;
        p.mode = md;
        p.prefix = pf;
        p.n_seg = n;
      }
      if (f == FMASK_TREE) {
        int32_t* par = at<int32_t>(out, L.parent);
        int32_t* hi = at<int32_t>(out, L.tree_hi);
        p.tree_prefix = desc->tree_prefix;
        p.tree_hi = hi;
        if (desc->tree_n > 0) {
          e = hipMemcpyAsync(par, desc->tree_parent, (size_t)desc->tree_n * sizeof(int32_t),
                             hipMemcpyHostToDevice, s);
          if (e != hipSuccess) return hip_status(e, "copy tree_parent");
          e = launch_tree_hi(par, desc->tree_n, hi, s);
          if (e != hipSuccess) return hip_status(e, "tree kernel");
        }
      }
      e = launch_encode_family_intervals(p, iv, s);
    }
    return hip_status(e, "encode kernel");
  }
  if (kind == FMASK_ENC_BITMAP) {
    BitmapSrc src{};
    src.nmask = nmask;
    src.nbq = (int32_t)L.nbq;
    src.nbk = (int32_t)L.nbk;
    src.sq = sq;
    src.skv = skv;
    if (f == FMASK_TREE) {
      src.kind = 1;
      src.tree_prefix = desc->tree_prefix;
      src.tree_n = desc->tree_n;
      int32_t* par = at<int32_t>(out, L.parent);
      if (desc->tree_n > 0) {
        e = hipMemcpyAsync(par, desc->tree_parent, (size_t)desc->tree_n * sizeof(int32_t),
                           hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_status(e, "copy tree_parent");
      }
      src.parent = par;
    } else if (f == FMASK_DENSE) {
      src.kind = 2;
      src.dense = desc->dense;
      src.dense_vec = skv % 16 == 0 && (uintptr_t)desc->dense % 16 == 0;
    } else {
      src.kind = 0;
      src.state = desc->blk_state;
      src.index = desc->blk_index;
      src.bits = desc->blk_bits;
      src.pool_n = desc->blk_pool_n;
      src.force_diag = desc->force_diag != 0;
    }
    BitmapOut o{};
    o.state = at<uint8_t>(out, L.bstate);
    o.index = at<int32_t>(out, L.bindex);
    o.bits = at<uint64_t>(out, L.bbits);
    o.cap = L.cap;
    o.row_count = at<int32_t>(out, L.row_count);
    o.row_offset = at<int32_t>(out, L.row_offset);
    o.pool_count = at<int32_t>(out, L.pool_count);
    enc->blk = kBlk;
    enc->blk_state = o.state;
    enc->blk_index = o.index;
    enc->blk_bits = o.bits;
    enc->blk_pool_count = o.pool_count;
    enc->nbq = L.nbq;
    enc->nbk = L.nbk;
    enc->pool_cap = L.cap;
    if (L.nbq * L.nbk == 0) {
      e = launch_zero_int(o.pool_count, s);
      return hip_status(e, "clear pool count");
    }
    e = launch_encode_bitmap(src, o, s);
    return hip_status(e, "bitmap encode kernels");
  }
  // SELECTED
  int32_t* list = at<int32_t>(out, L.list);
  int32_t* count = at<int32_t>(out, L.count);
  const int64_t nblk = ceil_div(desc->skv, desc->sel_cells);
  enc->blk = desc->sel_cells;
  enc->sel_list = list;
  enc->sel_count = count;
  enc->sel_n = desc->sel_n;
  e = launch_encode_selected(desc->sel, desc->batch, sq, desc->sel_n, (int32_t)nblk, list, count, s);
  return hip_status(e, "selected-key encode kernel");
}

size_t fmask_classify_bytes(const fmask_encoded* enc, int32_t bm, int32_t bn) {
  if (check_tiles_args(enc, bm, bn) != FMASK_OK) return 0;
  return tile_layout(enc, bm, bn).total;
}

fmask_status fmask_classify(const fmask_encoded* enc, int32_t bm, int32_t bn, void* out, size_t out_bytes,
                            fmask_tiles* tiles, void* stream) {
  g_err[0] = 0;
  fmask_status st = check_tiles_args(enc, bm, bn);
  if (st == FMASK_OK) st = check_mask_data(enc);
  if (st != FMASK_OK) return st;
  if (!tiles) return fail(FMASK_ERR_INVALID, "null fmask_tiles");
  if (!out || ((uintptr_t)out % kAlign)) return fail(FMASK_ERR_INVALID, "out must be 256-byte aligned");
  const TileLayout T = tile_layout(enc, bm, bn);
  if (out_bytes < T.total) return fail(FMASK_ERR_CAPACITY, "out has %zu bytes, %zu needed", out_bytes, T.total);
  hipStream_t s = (hipStream_t)stream;
  memset(tiles, 0, sizeof(*tiles));
  tiles->bm = bm;
  tiles->bn = bn;
  tiles->nqt = (int32_t)T.nqt;
  tiles->nkt = (int32_t)T.nkt;
  tiles->batch = enc->batch;
  tiles->heads = enc->heads;
  uint8_t* state = at<uint8_t>(out, T.state);
  int32_t* list = at<int32_t>(out, T.list);
  int32_t* count = at<int32_t>(out, T.count);
  int32_t* order = at<int32_t>(out, T.order);
  tiles->state = state;
  tiles->list = list;
  tiles->count = count;
  tiles->order = order;
  const int32_t nmask = (int32_t)((int64_t)enc->batch * enc->heads);  // rows <= 2^31 - 1 (check_tiles_args)
  hipError_t e;
  if (enc->kind == FMASK_ENC_INTERVALS)
    e = launch_classify_intervals(enc->intervals, nmask, (int32_t)enc->sq, (int32_t)enc->skv, bm, bn,
                                  (int32_t)T.nqt, (int32_t)T.nkt, state, s);
  else
    e = launch_classify_bitmap(enc->blk_state, nmask, (int32_t)enc->nbq, (int32_t)enc->nbk, bm, bn,
                               (int32_t)T.nqt, (int32_t)T.nkt, state, s);
  if (e != hipSuccess) return hip_status(e, "classify kernel");
  e = launch_tile_lists(state, (int32_t)T.rows, (int32_t)T.nkt, list, count, s);
  if (e != hipSuccess) return hip_status(e, "tile list kernel");
  e = launch_tile_order(count, (int32_t)T.rows, (int32_t)T.nqt, order, s);
  return hip_status(e, "tile order kernel");
}

fmask_status fmask_attn_fwd(const fmask_attn_args* a, const void* q, const void* k, const void* v, void* o,
                            float* lse, const fmask_encoded* enc, const fmask_tiles* tiles, void* stream) {
  g_err[0] = 0;
  if (!a || !enc) return fail(FMASK_ERR_INVALID, "null args or encoding");
  if (a->dtype != FMASK_BF16 && a->dtype != FMASK_F32) return fail(FMASK_ERR_UNSUPPORTED, "dtype %d", a->dtype);
  if (a->b < 1 || a->hq < 1 || a->hkv < 1 || a->hq % a->hkv)
    return fail(FMASK_ERR_INVALID, "need b, hq, hkv >= 1 and hq %% hkv == 0");
  if (a->sq < 0 || a->skv < 0 || a->sq > kMaxSeq || a->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "sq / skv out of range");
  if (a->sq != enc->sq || a->skv != enc->skv) return fail(FMASK_ERR_INVALID, "sq / skv differ from the encoding");
  if (!(enc->batch == 1 || enc->batch == a->b)) return fail(FMASK_ERR_INVALID, "encoding batch must be 1 or b");
  if (!(enc->heads == 1 || enc->heads == a->hq)) return fail(FMASK_ERR_INVALID, "encoding heads must be 1 or hq");
  if (!present(a->sq, {q, o}) || !present(a->skv, {k, v})) return fail(FMASK_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FMASK_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  const int64_t vec = a->dtype == FMASK_BF16 ? 8 : 4;
  for (int i = 0; i < 3; ++i) {
    if (a->q_stride[i] % vec || a->k_stride[i] % vec || a->v_stride[i] % vec || a->o_stride[i] % vec)
      return fail(FMASK_ERR_UNSUPPORTED, "strides must be multiples of %lld elements", (long long)vec);
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || a->v_stride[i] < 0 || a->o_stride[i] < 0)
      return fail(FMASK_ERR_INVALID, "negative stride");
  }
  hipStream_t s = (hipStream_t)stream;
  const int32_t group = a->hq / a->hkv;

  if (enc->kind == FMASK_ENC_SELECTED) {
    SelAttnParams p{};
    const fmask_status st = selected_params(a, q, k, v, o, lse, enc, &p);
    if (st != FMASK_OK) return st;
    return hip_status(launch_attn_selected_bf16(p, a->d, 1, nullptr, s), "selected-key attention kernel");
  }

  if (!tiles) return fail(FMASK_ERR_INVALID, "tile table required for this encoding");
  int32_t bm = 0, bn = 0;
  if ((a->dtype != FMASK_BF16 && a->dtype != FMASK_F32) || (a->d != 64 && a->d != 128))
    return fail(FMASK_ERR_UNSUPPORTED, "tile kernels: d in {64, 128}");
  bm = tiles->bm;
  bn = tiles->bn;
  if (check_mask_data(enc) != FMASK_OK) return FMASK_ERR_INVALID;
  if (!tile_supported(a->dtype, enc->kind, bm, bn)) {
    int32_t pbm = 0, pbn = 0;
    preferred(a->dtype, a->d, enc->kind, &pbm, &pbn);
    return fail(FMASK_ERR_UNSUPPORTED, "no kernel for %dx%d tiles here (preferred: %dx%d)", bm, bn, pbm, pbn);
  }
  if (tiles->nqt != ceil_div(a->sq, bm) || tiles->nkt != ceil_div(a->skv, bn) ||
      tiles->batch != enc->batch || tiles->heads != enc->heads)
    return fail(FMASK_ERR_INVALID, "tile table does not match the encoding");
  if (a->dtype == FMASK_BF16) {  // 32-bit buffer offsets inside one (batch, K/V head)
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if ((a->skv + 64) * a->k_stride[2] * 2 > lim || (a->skv + 64) * a->v_stride[2] * 2 > lim)
      return fail(FMASK_ERR_UNSUPPORTED, "one K/V head must span less than 2 GiB");
  }
  TileAttnParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  memcpy(p.qs, a->q_stride, sizeof(p.qs));
  memcpy(p.ks, a->k_stride, sizeof(p.ks));
  memcpy(p.vs, a->v_stride, sizeof(p.vs));
  memcpy(p.os, a->o_stride, sizeof(p.os));
  p.b = a->b; p.hq = a->hq; p.hkv = a->hkv; p.group = group;
  p.sq = (int32_t)a->sq; p.skv = (int32_t)a->skv; p.scale = a->scale;
  p.list = tiles->list; p.count = tiles->count; p.order = tiles->order;
  p.nqt = tiles->nqt; p.nkt = tiles->nkt; p.bm = bm; p.bn = bn;
  p.mb = enc->batch; p.mh = enc->heads;
  const int64_t expand = (int64_t)(enc->batch == 1 ? a->b : 1) * (enc->heads == 1 ? a->hq : 1);
  const int64_t items = bounded_prod({(int64_t)enc->batch * enc->heads, tiles->nqt, expand}, INT32_MAX / 2);
  if (items < 0) return fail(FMASK_ERR_UNSUPPORTED, "grid too large");
  p.expand = (int32_t)expand;
  p.n_items = (int32_t)items;
  {
    // (K/V head, batch) sets dealt whole to the XCDs (o3 kernel) when they
    // split evenly, every XCD's share holds all batch masks alike, and one set
    // fills an XCD's workgroup slots (32 CUs x 3): with smaller sets the last
    // set's longest rows would start when the XCD is nearly done
    const int64_t sets = (int64_t)a->b * a->hkv;
    p.set_major = sets % kXcds == 0 && enc->heads == 1 && (enc->batch == 1 || (sets / kXcds) % a->b == 0) &&
                  (int64_t)tiles->nqt * group >= 96;
  }
  p.kind = enc->kind;
  p.iv = enc->intervals;
  p.bstate = enc->blk_state; p.bindex = enc->blk_index; p.bbits = enc->blk_bits; p.pool_cap = enc->pool_cap;
  p.nbq = (int32_t)enc->nbq; p.nbk = (int32_t)enc->nbk;
  if (a->sq == 0) return FMASK_OK;
  hipError_t e;
  if (a->dtype == FMASK_F32) e = launch_attn_tile_f32(p, a->d, s);
  else if (bm == 128 && (enc->kind == FMASK_ENC_INTERVALS || (enc->kind == FMASK_ENC_BITMAP && enc->pool_cap <= ((int64_t)1 << 22))))
    e = launch_attn_o3_bf16(p, a->d, s);
  else if (bm == 64 && enc->kind == FMASK_ENC_BITMAP && enc->pool_cap <= ((int64_t)1 << 22))
    e = launch_attn_pair_bf16(p, a->d, s);
  else e = launch_attn_tile_bf16(p, a->d, s);
  return hip_status(e, "attention kernel");
}

size_t fmask_attn_split_workspace_bytes(const fmask_attn_args* a, const fmask_encoded* enc, int32_t splits) {
  if (!a || !enc || enc->kind != FMASK_ENC_SELECTED || splits < 0 || a->b < 1 || a->hkv < 1 ||
      a->hq < 1 || a->hq % a->hkv || a->sq < 0 || a->sq > kMaxSeq)
    return 0;
  if (a->d < 1 || bounded_prod({(int64_t)a->hq * a->b, a->sq, 4}, kMaxBytes) < 0) return 0;
  const int32_t ns = splits == 0 ? auto_splits(a, enc->sel_n) : splits;
  // a partial (m, l, O) per (batch, query head, query, split): d + 2 floats
  const int64_t bytes = bounded_prod({(int64_t)a->hq * a->b, a->sq, ns, (int64_t)a->d + 2, 4}, kMaxBytes);
  return bytes < 0 ? 0 : std::max<size_t>((size_t)bytes, kAlign);
}

}  // extern "C"

namespace {

// Checks and launches of the split form; the partial states go to `workspace`
// (workspace_bytes long).  what_ws names the buffer in error messages.
fmask_status split_fwd(const fmask_attn_args* a, const void* q, const void* k, const void* v, void* o,
                       float* lse, const fmask_encoded* enc, int32_t splits, void* workspace,
                       size_t workspace_bytes, const char* what_ws, void* stream) {
  if (!a || !enc) return fail(FMASK_ERR_INVALID, "null args or encoding");
  if (enc->kind != FMASK_ENC_SELECTED) return fail(FMASK_ERR_UNSUPPORTED, "split form: SELECTED encoding only");
  if (splits < 0 || splits > 64) return fail(FMASK_ERR_INVALID, "splits must be in [0, 64] (0 = automatic)");
  if (a->b < 1 || a->hq < 1 || a->hkv < 1 || a->hq % a->hkv)
    return fail(FMASK_ERR_INVALID, "need b, hq, hkv >= 1 and hq %% hkv == 0");
  if (a->sq < 0 || a->skv < 0 || a->sq > kMaxSeq || a->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "sq / skv out of range");
  if (a->sq != enc->sq || a->skv != enc->skv) return fail(FMASK_ERR_INVALID, "sq / skv differ from the encoding");
  if (!(enc->batch == 1 || enc->batch == a->b)) return fail(FMASK_ERR_INVALID, "encoding batch must be 1 or b");
  if (!present(a->sq, {q, o}) || !present(a->skv, {k, v})) return fail(FMASK_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FMASK_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (a->q_stride[i] % 8 || a->k_stride[i] % 8 || a->v_stride[i] % 8 || a->o_stride[i] % 8)
      return fail(FMASK_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || a->v_stride[i] < 0 || a->o_stride[i] < 0)
      return fail(FMASK_ERR_INVALID, "negative stride");
  }
  SelAttnParams p{};
  const fmask_status st = selected_params(a, q, k, v, o, lse, enc, &p);
  if (st != FMASK_OK) return st;
  const int32_t ns = splits == 0 ? auto_splits(a, enc->sel_n) : splits;
  const size_t need = fmask_attn_split_workspace_bytes(a, enc, ns);
  if (need == 0) return fail(FMASK_ERR_UNSUPPORTED, "split form: partial states would exceed 2^44 bytes");
  if (ns > 1) {
    if (!workspace || ((uintptr_t)workspace % 16)) return fail(FMASK_ERR_INVALID, "%s must be 16-byte aligned", what_ws);
    if (workspace_bytes < need)
      return fail(FMASK_ERR_CAPACITY, "%s has %zu bytes, %zu needed", what_ws, workspace_bytes, need);
  }
  return hip_status(launch_attn_selected_bf16(p, a->d, ns, (float*)workspace, (hipStream_t)stream),
                    "selected-key split kernels");
}

// Scratch area of the no-allocation split form: part of the library's code
// object, so every GPU the library runs on holds one copy for the life of the
// process.  Host code never uses the array's name as an address: its device
// address is looked up once per device (scratch_on_current_device) and that
// pointer is what the kernels receive.
static __device__ __align__(256) float scratch[FMASK_SPLIT_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

fmask_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FMASK_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(split scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FMASK_OK;
}

}  // namespace

extern "C" {

fmask_status fmask_attn_fwd_split(const fmask_attn_args* a, const void* q, const void* k, const void* v,
                                  void* o, float* lse, const fmask_encoded* enc, int32_t splits,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return split_fwd(a, q, k, v, o, lse, enc, splits, workspace, workspace_bytes, "workspace", stream);
}

fmask_status fmask_attn_fwd_split_noalloc(const fmask_attn_args* a, const void* q, const void* k, const void* v,
                                          void* o, float* lse, const fmask_encoded* enc, int32_t splits,
                                          void* stream) {
  g_err[0] = 0;
  if (!a || !enc) return fail(FMASK_ERR_INVALID, "null args or encoding");
  void* ws = nullptr;
  const fmask_status st = scratch_on_current_device(&ws);
  if (st != FMASK_OK) return st;
  return split_fwd(a, q, k, v, o, lse, enc, splits, ws, FMASK_SPLIT_SCRATCH_BYTES, "the library's split scratch",
                   stream);
}

size_t fmask_attn_blocks_workspace_bytes(const fmask_attn_args* a, const fmask_encoded* enc) {
  if (!a || !enc || enc->kind != FMASK_ENC_SELECTED || a->b < 1 || a->hkv < 1 || a->hq < 1 ||
      a->hq % a->hkv || a->sq < 0 || a->sq > kMaxSeq || a->skv < 0 || a->skv > kMaxSeq ||
      (a->d != 128 && a->d != 256) || enc->sel_n < 0 || enc->sel_n > FMASK_MAX_SEL_N || enc->batch < 1)
    return 0;
  if (bounded_prod({(int64_t)a->b * a->hq, a->sq, enc->sel_n, 2 * a->d + 8}, kMaxBytes) < 0) return 0;
  SelAttnParams p{};
  p.b = a->b; p.hq = a->hq; p.hkv = a->hkv; p.sq = (int32_t)a->sq; p.skv = (int32_t)a->skv;
  p.n = enc->sel_n; p.mb = enc->batch;
  return std::max<size_t>(selected_blocks_layout(p, a->d).total, kAlign);
}

fmask_status fmask_attn_fwd_blocks(const fmask_attn_args* a, const void* q, const void* k, const void* v,
                                   void* o, float* lse, const fmask_encoded* enc, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (!a || !enc) return fail(FMASK_ERR_INVALID, "null args or encoding");
  if (enc->kind != FMASK_ENC_SELECTED) return fail(FMASK_ERR_UNSUPPORTED, "block-major form: SELECTED encoding only");
  if (a->b < 1 || a->hq < 1 || a->hkv < 1 || a->hq % a->hkv)
    return fail(FMASK_ERR_INVALID, "need b, hq, hkv >= 1 and hq %% hkv == 0");
  if (a->sq < 0 || a->skv < 0 || a->sq > kMaxSeq || a->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "sq / skv out of range");
  if (a->sq != enc->sq || a->skv != enc->skv) return fail(FMASK_ERR_INVALID, "sq / skv differ from the encoding");
  if (!(enc->batch == 1 || enc->batch == a->b)) return fail(FMASK_ERR_INVALID, "encoding batch must be 1 or b");
  if (a->sq >= ((int64_t)1 << 23)) return fail(FMASK_ERR_UNSUPPORTED, "block-major form: fewer than 2^23 queries");
  // (the merge gives each list entry one lane of a wave; an encoding filled in
  // by hand must keep fmask_encode's limit)
  if (enc->sel_n < 1 || enc->sel_n > FMASK_MAX_SEL_N)
    return fail(FMASK_ERR_INVALID, "sel_n must be in [1, %d]", FMASK_MAX_SEL_N);
  if (!present(a->sq, {q, o}) || !present(a->skv, {k, v})) return fail(FMASK_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FMASK_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (a->q_stride[i] % 8 || a->k_stride[i] % 8 || a->v_stride[i] % 8 || a->o_stride[i] % 8)
      return fail(FMASK_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || a->v_stride[i] < 0 || a->o_stride[i] < 0)
      return fail(FMASK_ERR_INVALID, "negative stride");
  }
  {  // 32-bit buffer offsets inside one (batch, K/V head)
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if ((a->skv + 32) * a->k_stride[2] * 2 > lim || (a->skv + 32) * a->v_stride[2] * 2 > lim)
      return fail(FMASK_ERR_UNSUPPORTED, "one K/V head must span less than 2 GiB");
  }
  SelAttnParams p{};
  const fmask_status st = selected_params(a, q, k, v, o, lse, enc, &p);
  if (st != FMASK_OK) return st;
  const size_t need = fmask_attn_blocks_workspace_bytes(a, enc);
  if (need == 0) return fail(FMASK_ERR_UNSUPPORTED, "block-major form: partial states would exceed 2^44 bytes");
  if (!workspace || ((uintptr_t)workspace % 256)) return fail(FMASK_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(FMASK_ERR_CAPACITY, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(launch_attn_selected_blocks_bf16(p, a->d, workspace, (hipStream_t)stream),
                    "selected-key block-major kernels");
}

}  // extern "C"

namespace {
struct BwdLayout {
  size_t rows = 0, col_list = 0, col_count = 0, col_order = 0, total = 0;
  int64_t cols = 0;
};
BwdLayout bwd_layout(const fmask_attn_args* a, const fmask_tiles* t) {
  BwdLayout L;
  Carve c;
  L.cols = (int64_t)t->batch * t->heads * t->nkt;
  L.rows = c.take((size_t)a->b * a->hq * a->sq * 2 * sizeof(float));
  L.col_list = c.take((size_t)L.cols * t->nqt * sizeof(int32_t));
  L.col_count = c.take((size_t)L.cols * sizeof(int32_t));
  L.col_order = c.take((size_t)L.cols * sizeof(int32_t));
  L.total = std::max<size_t>(c.off, kAlign);
  return L;
}
}  // namespace

extern "C" {

size_t fmask_attn_bwd_workspace_bytes(const fmask_attn_args* a, const fmask_tiles* t) {
  if (!a || !t || a->b < 1 || a->hq < 1 || a->sq < 0 || a->sq > kMaxSeq || t->batch < 1 || t->heads < 1 ||
      t->nqt < 0 || t->nkt < 0)
    return 0;
  const int64_t cols = bounded_prod({(int64_t)t->batch * t->heads, t->nkt}, INT32_MAX);
  if (bounded_prod({(int64_t)a->b * a->hq, a->sq, 8}, kMaxBytes) < 0 || cols < 0 ||
      bounded_prod({cols, (int64_t)t->nqt + 2, 4}, kMaxBytes) < 0)
    return 0;
  return bwd_layout(a, t).total;
}

fmask_status fmask_attn_bwd(const fmask_attn_args* a, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dout, void* dq, void* dk,
                            void* dv, void* workspace, size_t workspace_bytes, const fmask_encoded* enc,
                            const fmask_tiles* tiles, void* stream) {
  g_err[0] = 0;
  if (!a || !enc || !tiles) return fail(FMASK_ERR_INVALID, "null args, encoding or tile table");
  if (a->dtype != FMASK_BF16) return fail(FMASK_ERR_UNSUPPORTED, "backward: bf16 only");
  if (a->d != 64 && a->d != 128) return fail(FMASK_ERR_UNSUPPORTED, "backward: d in {64, 128}");
  if (enc->kind != FMASK_ENC_INTERVALS && enc->kind != FMASK_ENC_BITMAP)
    return fail(FMASK_ERR_UNSUPPORTED, "backward: INTERVALS or BITMAP encodings");
  if (a->b < 1 || a->hq < 1 || a->hkv < 1 || a->hq % a->hkv)
    return fail(FMASK_ERR_INVALID, "need b, hq, hkv >= 1 and hq %% hkv == 0");
  if (a->sq < 0 || a->skv < 0 || a->sq > kMaxSeq || a->skv > kMaxSeq)
    return fail(FMASK_ERR_INVALID, "sq / skv out of range");
  if (a->sq != enc->sq || a->skv != enc->skv) return fail(FMASK_ERR_INVALID, "sq / skv differ from the encoding");
  if (!(enc->batch == 1 || enc->batch == a->b)) return fail(FMASK_ERR_INVALID, "encoding batch must be 1 or b");
  if (!(enc->heads == 1 || enc->heads == a->hq)) return fail(FMASK_ERR_INVALID, "encoding heads must be 1 or hq");
  if (tiles->bm != 128 || tiles->bn != 64)
    return fail(FMASK_ERR_UNSUPPORTED, "backward: tile table at 128 x 64 (have %d x %d)", tiles->bm, tiles->bn);
  if (tiles->nqt != ceil_div(a->sq, 128) || tiles->nkt != ceil_div(a->skv, 64) ||
      tiles->batch != enc->batch || tiles->heads != enc->heads)
    return fail(FMASK_ERR_INVALID, "tile table does not match the encoding");
  if (check_mask_data(enc) != FMASK_OK) return FMASK_ERR_INVALID;
  if (!present(a->sq, {q, o, lse, dout, dq}) || !present(a->skv, {k, v, dk, dv}))
    return fail(FMASK_ERR_INVALID, "null tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(FMASK_ERR_UNSUPPORTED, "tensors must be 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (a->q_stride[i] % 8 || a->k_stride[i] % 8 || a->v_stride[i] % 8 || a->o_stride[i] % 8)
      return fail(FMASK_ERR_UNSUPPORTED, "strides must be multiples of 8 elements");
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || a->v_stride[i] < 0 || a->o_stride[i] < 0)
      return fail(FMASK_ERR_INVALID, "negative stride");
  }
  const size_t need = fmask_attn_bwd_workspace_bytes(a, tiles);
  if (need == 0) return fail(FMASK_ERR_UNSUPPORTED, "backward: workspace would exceed 2^44 bytes");
  if (!workspace || ((uintptr_t)workspace % 16)) return fail(FMASK_ERR_INVALID, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FMASK_ERR_CAPACITY, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const int64_t lim = ((int64_t)1 << 31) - 1;  // 32-bit buffer offsets inside one head
  if ((a->skv + 64) * a->k_stride[2] * 2 > lim || (a->skv + 64) * a->v_stride[2] * 2 > lim ||
      (a->sq + 128) * a->q_stride[2] * 2 > lim || (a->sq + 128) * a->o_stride[2] * 2 > lim)
    return fail(FMASK_ERR_UNSUPPORTED, "one head must span less than 2 GiB");
  if (bounded_prod({(int64_t)a->b * a->hq, a->sq}, INT32_MAX / 4) < 0)
    return fail(FMASK_ERR_UNSUPPORTED, "problem too large");
  BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  memcpy(p.qs, a->q_stride, sizeof(p.qs));
  memcpy(p.ks, a->k_stride, sizeof(p.ks));
  memcpy(p.vs, a->v_stride, sizeof(p.vs));
  memcpy(p.os, a->o_stride, sizeof(p.os));
  p.b = a->b; p.hq = a->hq; p.hkv = a->hkv; p.group = a->hq / a->hkv;
  p.sq = (int32_t)a->sq; p.skv = (int32_t)a->skv; p.scale = a->scale;
  const BwdLayout L = bwd_layout(a, tiles);
  if (L.cols > INT32_MAX / 4) return fail(FMASK_ERR_UNSUPPORTED, "tile table too large");
  p.list = tiles->list; p.count = tiles->count; p.order = tiles->order;
  p.ws = at<float>(workspace, L.rows);
  int32_t* col_list = at<int32_t>(workspace, L.col_list);
  int32_t* col_count = at<int32_t>(workspace, L.col_count);
  int32_t* col_order = at<int32_t>(workspace, L.col_order);
  p.col_list = col_list; p.col_count = col_count; p.col_order = col_order;
  p.nqt = tiles->nqt; p.nkt = tiles->nkt; p.bm = tiles->bm; p.bn = tiles->bn;
  p.mb = enc->batch; p.mh = enc->heads;
  p.kind = enc->kind;
  p.iv = enc->intervals;
  p.bstate = enc->blk_state; p.bindex = enc->blk_index; p.bbits = enc->blk_bits;
  p.nbq = (int32_t)enc->nbq; p.nbk = (int32_t)enc->nbk;
  hipStream_t s = (hipStream_t)stream;
  // the tile table by key-tile column, and its longest-first order
  hipError_t ec = launch_tile_cols(tiles->state, enc->batch * enc->heads, tiles->nqt, tiles->nkt, col_list,
                                   col_count, s);
  if (ec == hipSuccess) ec = launch_tile_order(col_count, (int32_t)L.cols, (int32_t)L.cols, col_order, s);
  if (ec != hipSuccess) return hip_status(ec, "tile column kernels");
  return hip_status(launch_attn_bwd_bf16(p, a->d, s), "attention backward kernels");
}

}  // extern "C"
