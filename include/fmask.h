/*
 * fmask.h -- C ABI of libfmask: forward pass of exact softmax attention under a
 * structured sparse mask that is handed over in compressed form (never as a dense
 * Sq x Skv boolean matrix), for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operation (web pages on mask-aware attention):
 *  - FlashMask rebuttal (arXiv 2410.01359 review response): the mask types (causal
 *    document, document, shared question), the split between "mask block size" and
 *    the kernel's "tiling block size", and the point that fully masked blocks must
 *    not be computed.
 *  - "Efficiently Dispatching Flash Attention For Partially Filled Attention Masks"
 *    (Binary Block Masking), abstract: block-level mask awareness, sequence packing
 *    and Medusa tree masks.
 *  - Ascend CANN "sparseMode" page: attenMask semantics (the QK^T product is masked
 *    where the mask is set), the preTokens/nextTokens band anchored at the lower
 *    right corner, and cumulative sequence-length arrays.
 *  - llama.cpp fork PR "vulkan: selected-key flash attention for QSA block
 *    selection": attention whose visibility is a per-query list of K/V blocks of 32
 *    cells, with invalid (-1) and duplicate entries skipped.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says (host).
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *  - The library never allocates or frees device memory; the caller owns every
 *    buffer and sizes it with the *_bytes queries.  All launches are asynchronous
 *    on `stream`; host arrays named in a descriptor are consumed before the call
 *    returns (they are copied into the caller's `out` buffer).
 *  - Errors that the host can detect (null pointers, bad sizes, inconsistent
 *    descriptors, unsupported dtype / head size / tile shape, undersized buffers)
 *    return a negative status BEFORE anything is launched.  A failed launch
 *    returns FMASK_ERR_HIP.  No combination that a kernel does not implement is
 *    ever served by a kernel that ignores the mask: it returns
 *    FMASK_ERR_UNSUPPORTED instead.
 *  - fmask_last_error() gives a human-readable detail of the last failure on the
 *    calling thread.
 *  - sq or skv may be 0.  The tensors of an empty sequence (Q, O, LSE, dO, dQ
 *    for sq = 0; K, V, dK, dV for skv = 0) may then be null, as empty device
 *    tensors are; every other tensor pointer must be non-null.  With skv = 0
 *    every row is empty: O = 0, LSE = -inf, dQ = 0; with sq = 0, dK = dV = 0.
 *  - Sizes: sq and skv at most 2^30, batch * heads at most 2^31 - 1 masks.  A
 *    problem whose encoding, tile table or workspace would exceed 2^44 bytes is
 *    refused with FMASK_ERR_UNSUPPORTED, and the matching *_bytes query returns
 *    0 for it (size arithmetic never wraps).
 */
#ifndef FMASK_H
#define FMASK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t fmask_status;
#define FMASK_OK               0
#define FMASK_ERR_INVALID     (-1) /* inconsistent or out-of-range argument        */
#define FMASK_ERR_UNSUPPORTED (-2) /* valid, but no kernel implements it           */
#define FMASK_ERR_CAPACITY    (-3) /* a caller buffer is smaller than required     */
#define FMASK_ERR_HIP         (-4) /* the HIP runtime reported an error            */

/* Mask families.  vis(i, j) = 1 means query row i attends to key column j.
 * Row and column indices are 0-based token positions.                         */
enum fmask_family {
  /* j <= i (anchored at the upper left corner, Ascend "leftUpCausal").          */
  FMASK_CAUSAL = 1,
  /* seg(i) == seg(j), segments given by cu_seg (requires sq == skv).            */
  FMASK_DOCUMENT = 2,
  /* seg(i) == seg(j) and j <= i: packed sequences (FlashMask "causal document"). */
  FMASK_CAUSAL_DOCUMENT = 3,
  /* Segment 0 of cu_seg is the question, segments 1.. are answers:
   * j <= i and (seg(j) == seg(i) or seg(j) == 0)  (FlashMask "shared question"). */
  FMASK_SHARED_QUESTION = 4,
  /* Ascend band, anchored at the lower right corner:
   * with r = i + skv - sq:  r - pre_tokens <= j <= r + next_tokens (inclusive).
   * Negative pre_tokens or next_tokens are allowed; rows may become empty.      */
  FMASK_BAND = 5,
  /* Causal prefix of tree_prefix tokens followed by tree_n draft tokens whose
   * parents are tree_parent[t] (< t, -1 for a root).  Prefix rows are causal; a
   * draft row sees the whole prefix and its own ancestors and itself
   * (Medusa-style tree mask).  Requires sq == skv == tree_prefix + tree_n.      */
  FMASK_TREE = 6,
  /* 64 x 64 block pattern: per block SKIP / PARTIAL / FULL, PARTIAL blocks carry
   * 64 row words (bit c of word r = element (64*bi + r, 64*bj + c)); if
   * force_diag, every element (i, i) is visible as well (Binary Block Masking).  */
  FMASK_BLOCK_BITMAP = 7,
  /* Per query a list of sel_n block indices of sel_cells cells; a key is visible
   * iff its block floor(j / sel_cells) is listed.  Entries outside
   * [0, ceil(skv / sel_cells)) are ignored; duplicates count once.  No causal
   * term (visibility lives only in the list).                                   */
  FMASK_SELECTED_KEY = 8,
  /* Raw per-key-column masked row intervals [UTS, UTE) and [LTS, LTE) (the
   * FlashMask column encoding): element (i, j) is masked iff
   * UTS_j <= i < UTE_j or LTS_j <= i < LTE_j.                                   */
  FMASK_INTERVALS = 9,
  /* j <= i + skv - sq (anchored at the lower right corner, "rightDownCausal"). */
  FMASK_CAUSAL_BOTTOM_RIGHT = 10,
  /* Packed variable-length batch (Ascend "actual_seq_qlen / actual_seq_kvlen"):
   * query rows [cu_seg[s], cu_seg[s+1]) attend only to key columns
   * [cu_seg_k[s], cu_seg_k[s+1]) of the same segment s, under the segment's
   * mode seg_mode[s] (fmask_varlen_mode), with ii, jj the row / column inside
   * the segment and off = (segment keys) - (segment queries).               */
  FMASK_VARLEN = 11,
  /* Dense visibility given element by element: uint8 dense[batch][heads][sq][skv]
   * (device, row-major, nonzero = visible) -- the "allMask" input of the
   * Ascend sparseMode page, or Binary Block Masking's full mask.  Encoded into
   * the interval form when every column has at most two masked runs, else
   * into the 64 x 64 bitmap form (see dense_form).                            */
  FMASK_DENSE = 12
};

/* Per-segment modes of FMASK_VARLEN. */
enum fmask_varlen_mode {
  FMASK_VL_FULL = 0,                /* every (ii, jj)                                 */
  FMASK_VL_CAUSAL = 1,              /* jj <= ii        (upper left, "leftUpCausal")   */
  FMASK_VL_CAUSAL_BOTTOM_RIGHT = 2, /* jj <= ii + off  (lower right, "rightDownCausal") */
  FMASK_VL_BAND = 3,                /* r - pre_tokens <= jj <= r + next_tokens, r = ii + off */
  FMASK_VL_PREFIX = 4               /* jj < seg_prefix[s] or jj <= ii + off ("prefix") */
};

/* Kinds of canonical encoding written by fmask_encode. */
enum fmask_kind {
  FMASK_ENC_INTERVALS = 1, /* int32 SoA [batch][heads][4][skv]: UTS, UTE, LTS, LTE */
  FMASK_ENC_BITMAP    = 2, /* 64 x 64 block states + canonical word pool          */
  FMASK_ENC_SELECTED  = 3  /* sorted, de-duplicated, validated block lists        */
};

/* Tile-state byte values. */
enum fmask_tile_state { FMASK_SKIP = 0, FMASK_PARTIAL = 1, FMASK_FULL = 2 };

enum fmask_dtype { FMASK_F32 = 0, FMASK_BF16 = 1 };

#define FMASK_BLOCK          64          /* granularity of the bitmap encoding */
#define FMASK_LIST_FULL_BIT  0x80000000u /* flag in tile lists: tile is FULL   */
#define FMASK_MAX_SEL_N      64          /* longest selected-key list          */

/* Mask description (host struct).  Only the fields of `family` are read.
 *
 * batch / heads: number of distinct masks along the batch axis / query-head
 *   axis.  1 means one mask shared by every batch entry / head.  The segment,
 *   band, causal and tree families describe one mask (batch = heads = 1).
 *   FMASK_BLOCK_BITMAP and FMASK_INTERVALS accept batch >= 1 and heads >= 1;
 *   FMASK_SELECTED_KEY accepts batch >= 1 and heads == 1 (one list per query,
 *   shared by all heads).                                                       */
typedef struct fmask_mask_desc {
  int32_t family;
  int32_t batch;
  int32_t heads;
  int32_t reserved0;
  int64_t sq, skv;
  /* segment families: (host) cumulative boundaries cu_seg[0] = 0 <
   * cu_seg[1] < ... < cu_seg[n_seg] = sq; n_seg >= 1 segments.                  */
  const int32_t *cu_seg;
  int32_t n_seg;
  int32_t reserved1;
  /* band */
  int64_t pre_tokens, next_tokens;
  /* tree: (host) tree_parent[tree_n]                                            */
  const int32_t *tree_parent;
  int32_t tree_prefix, tree_n;
  /* block bitmap (device): blk_state uint8 [batch][heads][nbq][nbk] with
   * nbq = ceil(sq / 64), nbk = ceil(skv / 64); blk_index int32 same shape (pool
   * entry of a PARTIAL block, ignored otherwise); blk_bits [blk_pool_n][64].     */
  const uint8_t *blk_state;
  const int32_t *blk_index;
  const uint64_t *blk_bits;
  int64_t blk_pool_n;
  int32_t force_diag;
  int32_t reserved2;
  /* selected key (device): sel int32 [batch][sq][sel_n], sel_n <= 64.           */
  const int32_t *sel;
  int32_t sel_n, sel_cells;
  /* raw intervals (device): int32 [batch][heads][4][skv] in the order
   * UTS, UTE, LTS, LTE.                                                         */
  const int32_t *raw_intervals;
  /* varlen: (host) cu_seg holds the cumulative query lengths (n_seg + 1
   * entries, from 0 to sq, non-decreasing), cu_seg_k the cumulative key
   * lengths (from 0 to skv), seg_mode[n_seg] the modes, seg_prefix[n_seg] the
   * prefix widths (read for FMASK_VL_PREFIX segments only; may be NULL if
   * there is none); pre_tokens / next_tokens serve FMASK_VL_BAND segments.      */
  const int32_t *cu_seg_k;
  const int32_t *seg_mode;
  const int32_t *seg_prefix;
  /* dense (device): uint8 [batch][heads][sq][skv]; dense_form selects the
   * encoding: FMASK_ENC_BITMAP (always possible, asynchronous),
   * FMASK_ENC_INTERVALS (FMASK_ERR_INVALID if a column has more than two
   * masked runs), or 0 = the interval form when possible, else the bitmap
   * form.  The last two read one flag back from the device, i.e. they
   * synchronise `stream` (the only entry point that does).                      */
  const uint8_t *dense;
  int32_t dense_form;
  int32_t reserved3;
} fmask_mask_desc;

/* Canonical encoding (host struct filled by fmask_encode; device views into the
 * caller's `out` buffer, valid while that buffer lives).
 *
 * INTERVALS: for each (b, h, column j) the masked rows of column j, split into
 *   maximal runs: no run -> UT = [0,0), LT = [sq,sq); one run [a,b) -> UT = [0,b)
 *   if a == 0 else LT = [a,b) (the other one empty as above); two runs -> UT =
 *   the first, LT = the second.  Columns that would need more than two runs are
 *   not representable; fmask_encode then writes the BITMAP kind (tree family).
 * BITMAP: blk_state recomputed from the words (all valid elements set -> FULL,
 *   none -> SKIP), blk_index = -1 unless PARTIAL, pool entries in row-major
 *   (b, h, bi, bj) order, bits outside [0,sq) x [0,skv) cleared.
 * SELECTED: per (b, query) the valid distinct entries in ascending order,
 *   padded with -1 to sel_n, and their count.                                   */
typedef struct fmask_encoded {
  int32_t kind;
  int32_t batch, heads;
  int32_t blk;                     /* 64 (BITMAP) or sel_cells (SELECTED)       */
  int64_t sq, skv;
  const int32_t *intervals;        /* INTERVALS: [batch][heads][4][skv]         */
  const uint8_t *blk_state;        /* BITMAP: [batch][heads][nbq][nbk]          */
  const int32_t *blk_index;        /* BITMAP: same shape                        */
  const uint64_t *blk_bits;        /* BITMAP: [pool_cap][64]                    */
  const int32_t *blk_pool_count;   /* BITMAP: device scalar, entries used       */
  int64_t nbq, nbk, pool_cap;
  const int32_t *sel_list;         /* SELECTED: [batch][sq][sel_n]              */
  const int32_t *sel_count;        /* SELECTED: [batch][sq]                     */
  int32_t sel_n;
  int32_t reserved0;
} fmask_encoded;

/* Tile table (host struct filled by fmask_classify; device views into `out`).
 * Tile (qt, kt) covers rows [qt*bm, min((qt+1)*bm, sq)) and columns
 * [kt*bn, min((kt+1)*bn, skv)).  state is SKIP if no element of the tile is
 * visible, FULL if all are, PARTIAL otherwise (exact, element by element).
 * list[b][h][qt][0..count) holds the non-SKIP kt in ascending order, with
 * FMASK_LIST_FULL_BIT set for FULL tiles.  order[] lists the batch*heads*nqt
 * tile rows (index (b*heads + h)*nqt + qt): the nqt rows of mask slice (b, h)
 * occupy order[(b*heads + h)*nqt ...] in decreasing count, ties by index.      */
typedef struct fmask_tiles {
  int32_t bm, bn;
  int32_t nqt, nkt;
  int32_t batch, heads;
  int32_t reserved0, reserved1;
  const uint8_t *state;            /* [batch][heads][nqt][nkt]                  */
  const int32_t *list;             /* [batch][heads][nqt][nkt]                  */
  const int32_t *count;            /* [batch][heads][nqt]                       */
  const int32_t *order;            /* [batch*heads*nqt]                         */
} fmask_tiles;

/* Attention problem.  Q [b][hq][sq][d], K and V [b][hkv][skv][d], O like Q, in
 * `dtype` (FMASK_BF16: bfloat16, FMASK_F32: float); strides in elements for the
 * batch, head and sequence axes, the d axis is contiguous.  Query head h reads
 * K/V head h / (hq / hkv).  LSE (optional) is float [b][hq][sq], contiguous.   */
typedef struct fmask_attn_args {
  int32_t dtype;
  int32_t b, hq, hkv;
  int64_t sq, skv;
  int32_t d;
  int32_t reserved0;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  float scale;
  int32_t reserved1;
} fmask_attn_args;

/* Bytes of device memory fmask_encode needs for `desc`; 0 if desc is invalid. */
size_t fmask_encode_bytes(const fmask_mask_desc *desc);

/* Turn the mask description into its canonical compressed encoding (mask
 * encoder).  out: device buffer of at least fmask_encode_bytes(desc) bytes, 256-
 * byte aligned.  *enc (host) receives the kind and device views into out.
 * Defining passages: the FlashMask rebuttal (the mask types, and a mask kept
 * as a compact description instead of an Sq x Skv matrix whose size grows with
 * the sequence, "Response to Weaknesses and Questions"); the Ascend
 * "sparseMode" page (preTokens / nextTokens band and the cumulative-length
 * arrays of the varlen examples); the Binary Block Masking abstract (block
 * masks, packing, tree masks); the selected-key PR overview (per-query lists
 * of 32-cell blocks, -1 and duplicate entries skipped).
 * Host arrays: segment starts of up to 64 segments travel in kernel arguments;
 * larger cu_seg arrays, tree_parent and the varlen arrays are copied from the
 * caller's host memory with hipMemcpyAsync, which the HIP runtime stages before
 * the call returns (the caller may free them afterwards).  Those copies are not
 * safe under HIP graph capture (a captured copy would read the host array at
 * replay): capture only encodes of the other families.  The DENSE family in
 * the automatic or the interval form reads one flag back and synchronises the
 * stream (see dense_form).                                                      */
fmask_status fmask_encode(const fmask_mask_desc *desc, void *out, size_t out_bytes,
                          fmask_encoded *enc, void *stream);

/* Bytes of device memory fmask_classify needs; 0 if the arguments are invalid. */
size_t fmask_classify_bytes(const fmask_encoded *enc, int32_t bm, int32_t bn);

/* Reduce an INTERVALS or BITMAP encoding to the exact per-tile SKIP / PARTIAL /
 * FULL table at tile size bm x bn, plus per-row compact lists of the non-SKIP
 * tiles and a per-slice longest-first order of tile rows (tile classifier).
 * bm and bn are multiples of 16 in [16, 256]; the BITMAP kind needs multiples
 * of 64.
 * Defining passages: the FlashMask rebuttal ("Response to Weaknesses and
 * Questions": the kernel's tiling block size is separate from the mask's
 * block size, and fully masked blocks are not computed); the Binary Block
 * Masking abstract (blocks classified as empty, full or partially filled).
 * out: device buffer of fmask_classify_bytes(enc, bm, bn) bytes, 256-byte
 * aligned; *tiles (host) receives device views into out.  Kernels only: safe
 * under HIP graph capture.                                                      */
fmask_status fmask_classify(const fmask_encoded *enc, int32_t bm, int32_t bn, void *out,
                            size_t out_bytes, fmask_tiles *tiles, void *stream);

/* Defining passages: the FlashMask rebuttal ("Response to Weaknesses and
 * Questions": exact attention under the packed-sequence masks, fully masked
 * blocks skipped), the Ascend "sparseMode" page (attenMask: the scores QK^T
 * are masked where the mask is set, before the softmax), the Binary Block
 * Masking abstract, and the selected-key PR (visibility only from the list,
 * an empty list giving a zero row).
 * Masked attention forward: for every (batch, q head, row) with visible set V_i,
 * s_ij = scale * <Q_i, K_j>, O_i = sum_{j in V_i} softmax(s_i)_j V_j and
 * LSE_i = log sum_{j in V_i} exp(s_ij); a row with no visible key gets O_i = 0
 * and LSE_i = -inf.  SKIP tiles are never loaded, FULL tiles are computed
 * without per-element masking, PARTIAL tiles are masked element by element.
 * tiles must come from fmask_classify on the same encoding (NULL for the
 * SELECTED kind, whose kernel walks the lists directly).  Tile shapes with a
 * kernel: BF16 INTERVALS 128x64 (preferred), 256x64, 64x64; BF16 BITMAP 128x64
 * (preferred), 64x64; F32 64x64.  Other shapes return FMASK_ERR_UNSUPPORTED.
 * BF16 BITMAP at 128x64 walks, per 128-row tile, the key tiles where either
 * of its two 64-row blocks is non-empty (one K/V load serves both); at 64x64
 * a workgroup takes two block rows and each walks only its own non-empty
 * blocks, which suits sparse block patterns (few blocks shared by
 * neighbouring block rows: the Binary Block Masking abstract's extremely
 * sparse masks).
 * Supported: BF16 with d in {64, 128} on INTERVALS / BITMAP; F32 with d in
 * {64, 128} on INTERVALS / BITMAP; BF16 with d in {128, 256}, sel_cells == 32
 * and hq / hkv in {1, 2, 4, 8, 12, 16} on SELECTED.                             */
fmask_status fmask_attn_fwd(const fmask_attn_args *args, const void *q, const void *k,
                            const void *v, void *o, float *lse, const fmask_encoded *enc,
                            const fmask_tiles *tiles, void *stream);

/* Few-query (decode) form of fmask_attn_fwd for the SELECTED kind: each
 * query's list is split over `splits` workgroups (0 = automatic: enough to
 * cover the chip, at most one split per 4 entries), whose partial states
 * (running max m, sum l, unnormalised O per query head) go to `workspace` and
 * are merged by a second kernel with the split-K rule of the selected-key PR
 * (factors exp(m_s - max_s m_s); a split that sees no valid entry carries
 * m = -FLT_MAX, l = 0 and contributes nothing).  Same result as
 * fmask_attn_fwd up to rounding order; meant for a handful of queries, where
 * one workgroup per (query, K/V head) leaves the chip idle.  workspace: device
 * buffer of fmask_attn_split_workspace_bytes(args, enc, splits) bytes (unused
 * when the split count is 1).                                                  */
size_t fmask_attn_split_workspace_bytes(const fmask_attn_args *args, const fmask_encoded *enc,
                                        int32_t splits);
fmask_status fmask_attn_fwd_split(const fmask_attn_args *args, const void *q, const void *k,
                                  const void *v, void *o, float *lse, const fmask_encoded *enc,
                                  int32_t splits, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* The split form of fmask_attn_fwd_split for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc): the partial states go to a scratch area the library
 * holds on every GPU it runs on, FMASK_SPLIT_SCRATCH_BYTES long, instead of a
 * caller workspace.  Same arguments, checks and result as fmask_attn_fwd_split
 * (the same kernels run).  A problem whose partial states exceed the scratch
 * (fmask_attn_split_workspace_bytes(args, enc, splits) > FMASK_SPLIT_SCRATCH_
 * BYTES for splits > 1) returns FMASK_ERR_CAPACITY before any launch.  The
 * first call on a device looks the scratch address up (no allocation, no
 * stream operation).  Every call on a GPU shares that GPU's scratch and leaves
 * its partial states there: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.        */
#define FMASK_SPLIT_SCRATCH_BYTES ((size_t)16 << 20)
fmask_status fmask_attn_fwd_split_noalloc(const fmask_attn_args *args, const void *q, const void *k,
                                          const void *v, void *o, float *lse,
                                          const fmask_encoded *enc, int32_t splits, void *stream);

/* Bytes of device workspace fmask_attn_fwd_blocks needs; 0 if the arguments
 * are invalid.  About b * sq * sel_n * hq * (2 d + 8) bytes: a partial state
 * per (batch, query, list entry, query head).                                  */
size_t fmask_attn_blocks_workspace_bytes(const fmask_attn_args *args, const fmask_encoded *enc);

/* Block-major form of fmask_attn_fwd for the SELECTED kind, meant for many
 * queries (prefill over a selected-key context).  Defining passage: the
 * selected-key PR (visibility only from each query's list of 32-cell blocks,
 * an empty list giving a zero row; the split-K merge of partial states with
 * factors exp(m_s - max m), an empty part carrying m = -FLT_MAX).  Same
 * result as fmask_attn_fwd up to rounding: the lists are inverted into, per
 * block, the (query, entry) pairs that name it; each block's K and V are then
 * read once per K/V head and scored against the Q rows of those queries, which
 * gives one partial state (maximum, sum, O / sum rounded to bf16) per
 * (batch, query, head, entry) in `workspace`; a second kernel merges each
 * query's partials in entry order.  The result does not depend on the order
 * in which pairs reach a block.
 * Supported: BF16, d in {128, 256}, sel_cells == 32, hq / hkv in
 * {1, 2, 4, 8, 12, 16}, sq < 2^23, 1 <= sel_n <= FMASK_MAX_SEL_N (checked
 * here too, for encodings not made by fmask_encode: FMASK_ERR_INVALID).
 * workspace: device, 256-byte aligned, at
 * least fmask_attn_blocks_workspace_bytes(args, enc) bytes (else
 * FMASK_ERR_CAPACITY before any launch); its contents on entry do not
 * matter.  Kernels only, asynchronous on `stream`; calls that share a
 * workspace must be ordered by the caller.                                     */
fmask_status fmask_attn_fwd_blocks(const fmask_attn_args *args, const void *q, const void *k,
                                   const void *v, void *o, float *lse, const fmask_encoded *enc,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace fmask_attn_bwd needs: two floats per (batch, q
 * head, query row) and the tile table by key-tile column (per column the
 * non-SKIP query tiles, their count, and a longest-first order of the
 * columns); 0 if the arguments are invalid.                                   */
size_t fmask_attn_bwd_workspace_bytes(const fmask_attn_args *args, const fmask_tiles *tiles);

/* Gradient of fmask_attn_fwd (same args, encoding and tile table): given the
 * forward's output O and log-sum-exp LSE and the output gradient dO, writes
 * dQ, dK and dV.  With P_ij = exp(s_ij - LSE_i) on visible cells (0 elsewhere,
 * and for rows with LSE = -inf), D_i = sum_d dO_id O_id and
 * dS = P * (dO V^T - D):  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 * dK and dV summed over the query heads that share a K/V head.  This is the
 * analytic gradient of the forward's definition; training with packed or
 * structured masks is what the FlashMask rebuttal page builds the forward for.
 * Layouts: dQ like Q (q_stride), dK like K (k_stride), dV like V (v_stride),
 * O and dO share o_stride; LSE float [b][hq][sq] contiguous, as the forward
 * writes it.  workspace: device buffer of fmask_attn_bwd_workspace_bytes
 * bytes (16-byte aligned); its contents are rewritten by every call.
 * Supported: BF16, d in {64, 128}, INTERVALS or BITMAP encodings (every
 * family but selected-key lists; the bitmap form holds tree, block and dense
 * masks), the tile table at 128 x 64 (fmask_preferred_tile); otherwise
 * FMASK_ERR_UNSUPPORTED.                                                       */
fmask_status fmask_attn_bwd(const fmask_attn_args *args, const void *q, const void *k,
                            const void *v, const void *o, const float *lse, const void *dout,
                            void *dq, void *dk, void *dv, void *workspace,
                            size_t workspace_bytes, const fmask_encoded *enc,
                            const fmask_tiles *tiles, void *stream);

/* Tile shape the attention kernel for (dtype, d, encoding kind) uses. */
fmask_status fmask_preferred_tile(int32_t dtype, int32_t d, int32_t kind, int32_t *bm,
                                  int32_t *bn);

/* Static description of a status code. */
const char *fmask_status_str(fmask_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *fmask_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FMASK_H */
