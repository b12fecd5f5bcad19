/*
 * Host-side checks of libfmask's C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against a host-only build of the library (no
 * device code, no GPU): every call below returns from the library's own
 * argument checks, size arithmetic or host-array validation before anything
 * is launched or copied.  Covered: each mask family's descriptor with its host
 * arrays (segment starts, tree parents, varlen lengths, modes and prefixes)
 * read in full, malformed descriptors, sizes at and past the library's limits
 * (the size queries must refuse, never wrap), and the attention entry points'
 * argument checks.  Exit status 0 when every expectation holds; a sanitizer
 * report aborts the program.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fmask.h"

static int g_checks = 0, g_fail = 0;

#define EXPECT(cond, ...)                                  \
  do {                                                     \
    ++g_checks;                                            \
    if (!(cond)) {                                         \
      ++g_fail;                                            \
      fprintf(stderr, "FAIL line %d: ", __LINE__);         \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, " (last error: %s)\n", fmask_last_error()); \
    }                                                      \
  } while (0)

/* Never dereferenced: every call that receives it fails a host check first. */
#define DEV ((void *)(uintptr_t)0x100000)

static fmask_mask_desc desc(int32_t family, int64_t sq, int64_t skv) {
  fmask_mask_desc d;
  memset(&d, 0, sizeof(d));
  d.family = family;
  d.batch = 1;
  d.heads = 1;
  d.sq = sq;
  d.skv = skv;
  return d;
}

/* A descriptor the library accepts: its size query is positive, and encoding
 * into an empty buffer stops at the capacity check (host arrays already read). */
static void accepted(const fmask_mask_desc *d, const char *what) {
  fmask_encoded enc;
  const size_t need = fmask_encode_bytes(d);
  EXPECT(need >= 256, "%s: encode_bytes %zu", what, need);
  EXPECT(fmask_encode(d, DEV, 0, &enc, NULL) == FMASK_ERR_CAPACITY, "%s: capacity", what);
  EXPECT(fmask_encode(d, DEV, need - 1, &enc, NULL) == FMASK_ERR_CAPACITY, "%s: capacity - 1", what);
}

static void refused(const fmask_mask_desc *d, fmask_status want, const char *what) {
  fmask_encoded enc;
  EXPECT(fmask_encode_bytes(d) == 0, "%s: encode_bytes not 0", what);
  const fmask_status st = fmask_encode(d, DEV, (size_t)1 << 40, &enc, NULL);
  EXPECT(st == want, "%s: status %d, want %d", what, st, want);
  EXPECT(st == FMASK_OK || fmask_last_error()[0] != 0, "%s: no error text", what);
}

static void families(void) {
  /* parameter families */
  fmask_mask_desc d = desc(FMASK_CAUSAL, 1000, 1000);
  accepted(&d, "causal");
  d = desc(FMASK_CAUSAL_BOTTOM_RIGHT, 300, 1000);
  accepted(&d, "causal bottom right");
  d = desc(FMASK_BAND, 700, 900);
  d.pre_tokens = -20;
  d.next_tokens = -5;
  accepted(&d, "band, negative pre and next");
  d = desc(FMASK_CAUSAL, 0, 0);
  accepted(&d, "empty causal");

  /* segment families: cu_seg read to its last entry (here on the heap, so
   * that a read past it is an ASan report) */
  const int32_t cu_small[4] = {0, 100, 250, 400};
  int32_t *cu_big = malloc(sizeof(int32_t) * 301);
  for (int s = 0; s <= 300; ++s) cu_big[s] = 7 * s;
  const int fam[3] = {FMASK_DOCUMENT, FMASK_CAUSAL_DOCUMENT, FMASK_SHARED_QUESTION};
  for (int f = 0; f < 3; ++f) {
    d = desc(fam[f], 400, 400);
    d.cu_seg = cu_small;
    d.n_seg = 3;
    accepted(&d, "segments");
    d = desc(fam[f], 2100, 2100);
    d.cu_seg = cu_big;
    d.n_seg = 300;
    accepted(&d, "300 segments");
  }
  d = desc(FMASK_DOCUMENT, 400, 400);
  d.cu_seg = cu_small;
  d.n_seg = 3;
  d.skv = 401;
  refused(&d, FMASK_ERR_INVALID, "segments, sq != skv");
  d.skv = 400;
  const int32_t cu_flat[4] = {0, 100, 100, 400};
  d.cu_seg = cu_flat;
  refused(&d, FMASK_ERR_INVALID, "segments, empty segment");
  const int32_t cu_short[4] = {0, 100, 250, 399};
  d.cu_seg = cu_short;
  refused(&d, FMASK_ERR_INVALID, "segments, last != sq");
  d.cu_seg = NULL;
  refused(&d, FMASK_ERR_INVALID, "segments, no cu_seg");
  d.cu_seg = cu_small;
  d.batch = 2;
  refused(&d, FMASK_ERR_INVALID, "segments, batch 2");
  free(cu_big);

  /* tree: parents read in full, both encodings */
  const int n = 40;
  int32_t *par = malloc(sizeof(int32_t) * n);
  for (int t = 0; t < n; ++t) par[t] = t == 0 ? -1 : (t - 1) / 2;  /* BFS binary tree: not contiguous */
  d = desc(FMASK_TREE, 100 + n, 100 + n);
  d.tree_prefix = 100;
  d.tree_n = n;
  d.tree_parent = par;
  accepted(&d, "tree (bitmap form)");
  for (int t = 0; t < n; ++t) par[t] = t - 1;  /* a chain: every subtree contiguous */
  accepted(&d, "tree (interval form)");
  par[n - 1] = n - 1;
  refused(&d, FMASK_ERR_INVALID, "tree, parent not before its child");
  par[n - 1] = -2;
  refused(&d, FMASK_ERR_INVALID, "tree, parent < -1");
  free(par);
  d.tree_parent = NULL;
  refused(&d, FMASK_ERR_INVALID, "tree, no parents");
  d.tree_n = 5000;
  d.sq = d.skv = 5100;
  refused(&d, FMASK_ERR_INVALID, "tree, too many draft tokens");
  d = desc(FMASK_TREE, 64, 64);
  d.tree_prefix = 64;
  accepted(&d, "tree, no draft tokens");

  /* varlen: four host arrays */
  const int ns = 5;
  int32_t *cq = malloc(sizeof(int32_t) * (ns + 1)), *ck = malloc(sizeof(int32_t) * (ns + 1));
  int32_t *mode = malloc(sizeof(int32_t) * ns), *pre = malloc(sizeof(int32_t) * ns);
  const int32_t ql[5] = {100, 0, 37, 200, 63}, kl[5] = {120, 10, 37, 150, 0};
  cq[0] = ck[0] = 0;
  for (int s = 0; s < ns; ++s) {
    cq[s + 1] = cq[s] + ql[s];
    ck[s + 1] = ck[s] + kl[s];
    mode[s] = s % 5;
    pre[s] = 3 * s;
  }
  d = desc(FMASK_VARLEN, cq[ns], ck[ns]);
  d.cu_seg = cq;
  d.cu_seg_k = ck;
  d.seg_mode = mode;
  d.seg_prefix = pre;
  d.n_seg = ns;
  d.pre_tokens = 10;
  accepted(&d, "varlen");
  mode[2] = 7;
  refused(&d, FMASK_ERR_INVALID, "varlen, unknown mode");
  mode[2] = FMASK_VL_PREFIX;
  pre[2] = -1;
  refused(&d, FMASK_ERR_INVALID, "varlen, negative prefix");
  pre[2] = 0;
  d.seg_prefix = NULL;
  refused(&d, FMASK_ERR_INVALID, "varlen, prefix segment without prefixes");
  d.seg_prefix = pre;
  ck[3] = ck[2] - 1;
  refused(&d, FMASK_ERR_INVALID, "varlen, decreasing key lengths");
  ck[3] = ck[2] + kl[2];
  d.skv += 1;
  refused(&d, FMASK_ERR_INVALID, "varlen, keys do not end at skv");
  free(cq);
  free(ck);
  free(mode);
  free(pre);

  /* device-array families: pointers are only checked for presence here */
  d = desc(FMASK_BLOCK_BITMAP, 1000, 700);
  d.batch = 2;
  d.heads = 3;
  d.blk_state = DEV;
  d.blk_index = DEV;
  d.blk_bits = DEV;
  d.blk_pool_n = 10;
  accepted(&d, "block bitmap");
  d.blk_pool_n = -1;
  refused(&d, FMASK_ERR_INVALID, "block bitmap, negative pool");
  d = desc(FMASK_SELECTED_KEY, 2048, 131072);
  d.batch = 2;
  d.sel = DEV;
  d.sel_n = 64;
  d.sel_cells = 32;
  accepted(&d, "selected key");
  d.sel_n = 65;
  refused(&d, FMASK_ERR_INVALID, "selected key, 65 entries");
  d.sel_n = 64;
  d.heads = 2;
  refused(&d, FMASK_ERR_INVALID, "selected key, per-head lists");
  d = desc(FMASK_INTERVALS, 500, 600);
  d.batch = 3;
  d.heads = 2;
  d.raw_intervals = DEV;
  accepted(&d, "raw intervals");
  d.raw_intervals = NULL;
  refused(&d, FMASK_ERR_INVALID, "raw intervals missing");
  for (int form = 0; form <= 2; ++form) {
    d = desc(FMASK_DENSE, 300, 500);
    d.batch = 2;
    d.heads = 2;
    d.dense = DEV;
    d.dense_form = form == 0 ? 0 : (form == 1 ? FMASK_ENC_INTERVALS : FMASK_ENC_BITMAP);
    accepted(&d, "dense");
  }
  d.dense_form = 5;
  refused(&d, FMASK_ERR_INVALID, "dense, unknown form");

  d = desc(99, 10, 10);
  refused(&d, FMASK_ERR_INVALID, "unknown family");
  d = desc(FMASK_CAUSAL, -1, 10);
  refused(&d, FMASK_ERR_INVALID, "negative sq");
  d = desc(FMASK_CAUSAL, ((int64_t)1 << 30) + 1, 10);
  refused(&d, FMASK_ERR_INVALID, "sq past 2^30");
  EXPECT(fmask_encode_bytes(NULL) == 0, "null descriptor");
  d = desc(FMASK_CAUSAL, 10, 10);
  fmask_encoded enc;
  EXPECT(fmask_encode(&d, DEV, 1 << 20, NULL, NULL) == FMASK_ERR_INVALID, "null fmask_encoded");
  EXPECT(fmask_encode(&d, (void *)((uintptr_t)DEV + 16), 1 << 20, &enc, NULL) == FMASK_ERR_INVALID,
         "unaligned out");
}

/* Mask sizes past what any buffer could hold: the size queries refuse them
 * instead of wrapping, and so does every entry point. */
static void huge_masks(void) {
  const int64_t big = (int64_t)1 << 30;
  const int32_t many = 0x7fffffff;
  fmask_mask_desc d = desc(FMASK_INTERVALS, big, big);
  d.batch = many;
  d.heads = many;
  d.raw_intervals = DEV;
  refused(&d, FMASK_ERR_UNSUPPORTED, "intervals, 2^62 masks of 2^30 keys");
  d.batch = 1 << 12;
  d.heads = 1;
  refused(&d, FMASK_ERR_UNSUPPORTED, "intervals, 2^12 masks of 2^30 keys");
  d = desc(FMASK_BLOCK_BITMAP, big, big);
  d.batch = many;
  d.heads = many;
  d.blk_state = DEV;
  d.blk_index = DEV;
  refused(&d, FMASK_ERR_UNSUPPORTED, "block bitmap, 2^62 masks of 2^48 blocks");
  d.batch = d.heads = 1;
  refused(&d, FMASK_ERR_UNSUPPORTED, "block bitmap, one mask of 2^48 blocks");
  d = desc(FMASK_SELECTED_KEY, big, big);
  d.batch = many;
  d.sel = DEV;
  d.sel_n = 64;
  d.sel_cells = 32;
  refused(&d, FMASK_ERR_UNSUPPORTED, "selected key, 2^31 batches of 2^30 queries");
  d = desc(FMASK_DENSE, big, big);
  d.batch = many;
  d.heads = many;
  d.dense = DEV;
  refused(&d, FMASK_ERR_UNSUPPORTED, "dense, 2^62 masks");

  /* classify: hand-filled encodings with huge extents */
  fmask_encoded e;
  memset(&e, 0, sizeof(e));
  e.kind = FMASK_ENC_INTERVALS;
  e.batch = many;
  e.heads = many;
  e.sq = e.skv = big;
  e.intervals = DEV;
  fmask_tiles t;
  EXPECT(fmask_classify_bytes(&e, 16, 16) == 0, "classify_bytes, 2^62 masks");
  EXPECT(fmask_classify(&e, 16, 16, DEV, (size_t)1 << 62, &t, NULL) == FMASK_ERR_UNSUPPORTED,
         "classify, 2^62 masks");
  e.batch = e.heads = 1;
  EXPECT(fmask_classify_bytes(&e, 16, 16) == 0, "classify_bytes, 2^52 tiles");
  e.sq = e.skv = 1000;
  EXPECT(fmask_classify_bytes(&e, 128, 64) >= 256, "classify_bytes, ordinary");
  EXPECT(fmask_classify_bytes(&e, 100, 64) == 0, "classify_bytes, bm not a multiple of 16");
  EXPECT(fmask_classify(&e, 128, 64, DEV, 0, &t, NULL) == FMASK_ERR_CAPACITY, "classify, capacity");
  e.kind = FMASK_ENC_SELECTED;
  EXPECT(fmask_classify_bytes(&e, 128, 64) == 0, "classify_bytes, selected kind");
}

/* x * y, or 0 when the product does not fit (strides of the huge problems
 * below; a zero stride is valid and never multiplied on the host) */
static int64_t mul_or_0(int64_t x, int64_t y) {
  int64_t r;
  return __builtin_mul_overflow(x, y, &r) ? 0 : r;
}

static fmask_attn_args args(int64_t b, int64_t hq, int64_t hkv, int64_t sq, int64_t skv, int32_t d) {
  fmask_attn_args a;
  memset(&a, 0, sizeof(a));
  a.dtype = FMASK_BF16;
  a.b = (int32_t)b;
  a.hq = (int32_t)hq;
  a.hkv = (int32_t)hkv;
  a.sq = sq;
  a.skv = skv;
  a.d = d;
  a.scale = 0.125f;
  a.q_stride[0] = mul_or_0(hq, sq * d);
  a.q_stride[1] = sq * d;
  a.q_stride[2] = d;
  a.o_stride[0] = a.q_stride[0];
  a.o_stride[1] = a.q_stride[1];
  a.o_stride[2] = d;
  a.k_stride[0] = mul_or_0(hkv, skv * d);
  a.k_stride[1] = skv * d;
  a.k_stride[2] = d;
  memcpy(a.v_stride, a.k_stride, sizeof(a.k_stride));
  return a;
}

static void attention(void) {
  const int32_t many = 0x7fffffff;
  fmask_encoded iv;
  memset(&iv, 0, sizeof(iv));
  iv.kind = FMASK_ENC_INTERVALS;
  iv.batch = iv.heads = 1;
  iv.sq = iv.skv = 4096;
  iv.intervals = DEV;
  fmask_tiles t;
  memset(&t, 0, sizeof(t));
  t.bm = 128;
  t.bn = 64;
  t.nqt = 32;
  t.nkt = 64;
  t.batch = t.heads = 1;
  t.state = DEV;
  t.list = DEV;
  t.count = DEV;
  t.order = DEV;
  fmask_attn_args a = args(1, 8, 2, 4096, 4096, 128);
  float *lse = (float *)DEV;
  EXPECT(fmask_attn_fwd(NULL, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) == FMASK_ERR_INVALID, "fwd, null args");
  a.hq = 7;
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) == FMASK_ERR_INVALID, "fwd, hq %% hkv");
  a = args(1, 8, 2, 4096, 4096, 96);
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) == FMASK_ERR_UNSUPPORTED, "fwd, d 96");
  a = args(1, 8, 2, 4096, 4096, 128);
  a.q_stride[2] = 129;
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) == FMASK_ERR_UNSUPPORTED, "fwd, stride");
  a = args(1, 8, 2, 4096, 4096, 128);
  t.nqt = 31;
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) == FMASK_ERR_INVALID, "fwd, table size");
  t.nqt = 32;
  a = args(many, many, 1, (int64_t)1 << 30, (int64_t)1 << 30, 128);
  iv.sq = iv.skv = (int64_t)1 << 30;
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &t, NULL) < 0, "fwd, huge problem");
  /* a matching tile table over 64 keys: the check of the work-item count */
  a = args(many, many, 1, (int64_t)1 << 30, 64, 128);
  iv.skv = 64;
  fmask_tiles tb = t;
  tb.nqt = 1 << 23;
  tb.nkt = 1;
  EXPECT(fmask_attn_fwd(&a, DEV, DEV, DEV, DEV, lse, &iv, &tb, NULL) == FMASK_ERR_UNSUPPORTED,
         "fwd, 2^85 work items");
  iv.sq = iv.skv = 4096;

  /* selected-key forms: workspace queries refuse what cannot be sized */
  fmask_encoded sel;
  memset(&sel, 0, sizeof(sel));
  sel.kind = FMASK_ENC_SELECTED;
  sel.batch = sel.heads = 1;
  sel.blk = 32;
  sel.sq = 2048;
  sel.skv = 131072;
  sel.sel_list = DEV;
  sel.sel_count = DEV;
  sel.sel_n = 64;
  a = args(1, 16, 4, 2048, 131072, 256);
  const size_t ws_blocks = fmask_attn_blocks_workspace_bytes(&a, &sel);
  EXPECT(ws_blocks >= (size_t)2048 * 64 * 16 * (2 * 256 + 8), "blocks workspace %zu", ws_blocks);
  EXPECT(fmask_attn_fwd_blocks(&a, DEV, DEV, DEV, DEV, lse, &sel, DEV, ws_blocks - 1, NULL) == FMASK_ERR_CAPACITY,
         "blocks, capacity");
  EXPECT(fmask_attn_split_workspace_bytes(&a, &sel, 4) >= 256, "split workspace");
  EXPECT(fmask_attn_fwd_split(&a, DEV, DEV, DEV, DEV, lse, &sel, 65, DEV, 1 << 30, NULL) == FMASK_ERR_INVALID,
         "split, 65 splits");
  EXPECT(fmask_attn_fwd_split_noalloc(NULL, DEV, DEV, DEV, DEV, lse, &sel, 0, NULL) == FMASK_ERR_INVALID,
         "split no-alloc, null args");
  a = args(many, many, 1, (int64_t)1 << 30, (int64_t)1 << 30, 256);
  sel.sq = sel.skv = (int64_t)1 << 30;
  EXPECT(fmask_attn_blocks_workspace_bytes(&a, &sel) == 0, "blocks workspace, huge problem");
  EXPECT(fmask_attn_split_workspace_bytes(&a, &sel, 64) == 0, "split workspace, huge problem");
  a = args(1, 16, 4, 2048, 131072, 256);
  sel.sq = 2048;
  sel.skv = 131072;
  EXPECT(fmask_attn_split_workspace_bytes(&a, &sel, 0x7fffffff) == 0, "split workspace, 2^31 splits");
  a = args(1, 0x10000, 1, 2048, 131072, 256);
  EXPECT(fmask_attn_fwd_blocks(&a, DEV, DEV, DEV, DEV, lse, &sel, DEV, (size_t)1 << 50, NULL) ==
             FMASK_ERR_UNSUPPORTED,
         "blocks, 2^16 query heads per K/V head");

  /* backward */
  a = args(1, 8, 2, 4096, 4096, 128);
  const size_t ws_bwd = fmask_attn_bwd_workspace_bytes(&a, &t);
  EXPECT(ws_bwd >= (size_t)8 * 4096 * 8, "backward workspace %zu", ws_bwd);
  EXPECT(fmask_attn_bwd(&a, DEV, DEV, DEV, DEV, lse, DEV, DEV, DEV, DEV, DEV, ws_bwd - 16, &iv, &t, NULL) ==
             FMASK_ERR_CAPACITY,
         "backward, capacity");
  a = args(many, many, 1, (int64_t)1 << 30, (int64_t)1 << 30, 128);
  fmask_tiles th = t;
  th.batch = th.heads = many;
  th.nqt = th.nkt = many;
  EXPECT(fmask_attn_bwd_workspace_bytes(&a, &th) == 0, "backward workspace, huge problem");
}

int main(void) {
  families();
  huge_masks();
  attention();
  printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
