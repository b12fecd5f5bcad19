// Masked attention forward for block-bitmap masks at 64 x 64 tiles, bf16
// inputs, fp32 accumulation, gfx950 MFMA: a workgroup of four waves takes two
// 64-row block rows, and each pair of waves walks its own block row's list of
// non-empty blocks with its own K and V tiles in LDS.
//
// This is the schedule for sparse block masks (the Binary Block Masking
// abstract's "extremely sparse" case).  Under one 128-row tile the two 64-row
// blocks of a key tile are rarely both non-empty when blocks are sparse, so a
// 128-row kernel walks the union of the two block rows' lists with half of its
// waves idle at most steps, and the busy half uses two of the CU's four SIMDs.
// Here the halves step in lockstep through their own lists: max(|A|, |B|)
// steps instead of |A u B|, both halves busy until the shorter list ends.  The
// two block rows of a workgroup are consecutive in the longest-first order of
// their mask slice, so their list lengths are close.  When both halves' j-th
// entries name the same key tile (two rows of a causal or near-causal block
// pattern), the second half reads the first half's K and V tiles instead of
// loading its own, so such a tile is loaded once for 128 rows.
//
// The per-wave arithmetic is that of the 128-row kernel (attn_bf16_o3.hip):
// S^T = K Q^T with one query row per lane, bitmap row words as element masks,
// online softmax in the exp2 domain with a lazy running maximum, O^T += V^T P^T
// through the transposing LDS read.  LDS per workgroup (D = 128): per half one
// K and one V tile (4 x 16 KB), each wave's 32 row words of its block
// (4 x 256 B), per half the first kPList list entries and their block info
// (2 x 2 KB): 69 KB, two workgroups per CU.  Per step, each half:
//   issue V(j); QK(j), mask, softmax
//   barrier (K(j) and the row words read); issue K(j + 1) and its row words
//   wait V(j); barrier; PV(j)
//   wait for K(j + 1); barrier
#include <float.h>

#include "attn_common.h"
#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

constexpr int BN = 64;       // key tile (one bitmap block column)
constexpr int HR = 64;       // rows per half (one bitmap block row)
constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int kPList = 256;  // list entries per half staged in LDS

template <int D>
struct PGeo {
  static constexpr int KCH = D / 8;
  static constexpr int TILE = BN * D * 2;
  static constexpr int SLOT = 2 * TILE;                 // one half: K tile, then V tile
  static constexpr int WORDS = 2 * SLOT;                // row words [NW][32] uint64
  static constexpr int LST = WORDS + NW * 256;          // [2][kPList] key tile of each entry
  static constexpr int INFO = LST + 2 * kPList * 4;     // [2][kPList] block info of each entry
  static constexpr int END = INFO + 2 * kPList * 4;
  static constexpr int LOADS = BN * KCH / 128;          // 16-byte loads per wave and tile
  static_assert(BN * KCH % 128 == 0, "tile must split evenly over two waves");
  static_assert(TILE >= 2 * 4096, "epilogue staging: 4 KB per wave in its half's K tile");
};

struct PairItem {
  int b, h, kvh, mb, mh;
  int row0, row1;  // tile rows of the two halves (-1: none)
};

// Item l of the pair table: pairs of consecutive tile rows in the order of
// their mask slice (rows 2m and 2m + 1 of np = ceil(nqt / 2) pairs per slice),
// expanded over the (batch, head) pairs that share the slice.
//   set_major: l = ((kvh * b + batch) * np + m) * group + j, the blocks of
//              XCD x taking items [x n / 8, (x + 1) n / 8) so that an XCD works
//              through whole (K/V head, batch) sets in turn (L2 reuse of K, V);
//   otherwise: l = (slice * np + m) * expand + e, groups of gsz items dealt
//              round-robin over the XCDs.
__device__ inline bool pair_item(const TileAttnParams& p, int n_items, int set_major, int gsz,
                                 PairItem& it) {
  const int np = (p.nqt + 1) >> 1;
  int m;
  if (set_major) {
    const int per = n_items / kXcds, k = blockIdx.x / kXcds;
    if (k >= per) return false;
    const int l = (int)(blockIdx.x % kXcds) * per + k;
    const int j = l % p.group;
    int r = l / p.group;
    m = r % np;
    r /= np;
    it.b = r % p.b;
    it.kvh = r / p.b;
    it.h = it.kvh * p.group + j;
    it.mb = p.mb > 1 ? it.b : 0;
    it.mh = p.mh > 1 ? it.h : 0;
  } else {
    const int q = blockIdx.x;
    const int xcd = q % kXcds, k = q / kXcds;
    const int l = ((k / gsz) * kXcds + xcd) * gsz + (k % gsz);
    if (l >= n_items) return false;
    const int rp = l / p.expand, e = l % p.expand;
    const int slice = rp / np;
    m = rp % np;
    it.mb = slice / p.mh;
    it.mh = slice % p.mh;
    if (p.mb == 1 && p.mh == 1) { it.b = e / p.hq; it.h = e % p.hq; }
    else if (p.mb == 1) { it.b = e; it.h = it.mh; }
    else if (p.mh == 1) { it.b = it.mb; it.h = e; }
    else { it.b = it.mb; it.h = it.mh; }
    it.kvh = it.h / p.group;
  }
  const int base = (it.mb * p.mh + it.mh) * p.nqt;
  it.row0 = p.order[base + 2 * m];
  it.row1 = 2 * m + 1 < p.nqt ? p.order[base + 2 * m + 1] : -1;
  return true;
}

template <int D>
__global__ void __launch_bounds__(NT, D == 64 ? 3 : 2)
    k_attn_pair(TileAttnParams p, int n_items, int set_major, int gsz) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = PGeo<D>;
  constexpr int DB = D / 32;
  constexpr int KT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[G::END];

  PairItem it;
  if (!pair_item(p, n_items, set_major, gsz, it)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = w >> 1, wl = w & 1;  // half, wave within the half
  const int half = lane >> 5, l32 = lane & 31;
  const int row = hf ? it.row1 : it.row0;
  const int cnt0 = p.count[it.row0];
  const int cnt1 = it.row1 >= 0 ? p.count[it.row1] : 0;
  const int cnt = hf ? cnt1 : cnt0;
  const int steps = max(cnt0, cnt1);
  const int qt = row >= 0 ? row % p.nqt : 0;  // this half's block row
  const int r0 = qt * HR + wl * 32;           // first row of this wave
  const int qrow = r0 + l32;

  const __bf16* Q = (const __bf16*)p.q + it.b * p.qs[0] + it.h * p.qs[1];
  const __bf16* K = (const __bf16*)p.k + it.b * p.ks[0] + it.kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + it.b * p.vs[0] + it.kvh * p.vs[1];
  const int32_t* list = p.list + (int64_t)(row >= 0 ? row : 0) * p.nkt;
  const int32_t* list0 = p.list + (int64_t)it.row0 * p.nkt;
  const int32_t* list1 = p.list + (int64_t)(it.row1 >= 0 ? it.row1 : 0) * p.nkt;
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];

  // This half's first kPList list entries (key tile) and the block info of
  // each (pool index if PARTIAL, else kBlkFull / kBlkSkip), staged by its
  // 128 threads.  (LDS is not cleared: every byte a wave reads is written
  // first, K and V tiles entirely by their loads, zeros past the end included.)
  const size_t bbase = (((size_t)it.mb * p.mh + it.mh) * p.nbq + qt) * p.nbk;
  auto block_info = [&](int kt) INLINE -> int {
    const int st = p.bstate[bbase + kt];
    return st == FMASK_PARTIAL ? p.bindex[bbase + kt] : (st == FMASK_FULL ? kBlkFull : kBlkSkip);
  };
  int32_t* lst = (int32_t*)(smem + G::LST) + hf * kPList;
  int32_t* inf = (int32_t*)(smem + G::INFO) + hf * kPList;
  for (int i = tid & 127; i < min(cnt, kPList); i += 128) {
    const int kt = list[i] & 0x7fffffff;
    lst[i] = kt;
    inf[i] = block_info(kt);
  }
  // key tile of entry i of half h (both halves read both lists)
  auto kt_of = [&](int h, int i) INLINE -> int {
    if (i < kPList) return __builtin_amdgcn_readfirstlane(((const int32_t*)(smem + G::LST))[h * kPList + i]);
    return sload_wait((h ? list1 : list0) + i) & 0x7fffffff;
  };
  // both halves' j-th entries name the same key tile
  auto shared_at = [&](int i) INLINE -> bool {
    return i < cnt0 && i < cnt1 && kt_of(0, i) == kt_of(1, i);
  };
  // Past the staged entries the block info is read with scalar loads: a
  // vector load's wait would also drain the tile loads in flight.
  const int bbase_u = __builtin_amdgcn_readfirstlane((int)bbase);  // < 2^22 blocks (launcher)
  auto entry = [&](int i, int& kt, int& info) INLINE {
    if (i < kPList) {
      kt = __builtin_amdgcn_readfirstlane(lst[i]);
      info = __builtin_amdgcn_readfirstlane(inf[i]);
    } else {
      kt = sload_wait(list + i) & 0x7fffffff;
      const int st = sload_byte(p.bstate + bbase_u + kt);
      info = st == FMASK_PARTIAL ? sload_wait(p.bindex + bbase_u + kt) : (st == FMASK_FULL ? kBlkFull : kBlkSkip);
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = p.scale * kLog2e;

  const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);
  const rsrc_t irs = make_rsrc(p.bbits, p.pool_cap * kBlk * 8);
  // Direct-to-LDS loads: instruction n of wave wl of a half fills the chunks
  // P = (wl * LOADS + n) * 64 + lane of that half's tile, i.e. row P / KCH,
  // physical chunk P % KCH holding logical chunk (P % KCH) ^ swizzle(row).
  // The V swizzle does not depend on n (rows advance by a multiple of 4 per
  // instruction), so one lane offset serves all of V's loads.
  int kgo[G::LOADS];
#pragma unroll
  for (int n = 0; n < G::LOADS; ++n) {
    const int P = (wl * G::LOADS + n) * 64 + lane;
    const int key = P / G::KCH, pc = P % G::KCH;
    kgo[n] = (int)(key * ks2 * 2 + ((pc ^ kswz<G::KCH>(key)) * 16));
  }
  int vgo;
  {
    const int P = wl * G::LOADS * 64 + lane;
    const int key = P / G::KCH, pc = P % G::KCH;
    vgo = (int)(key * vs2 * 2 + ((pc ^ vswz<G::KCH>(key)) * 16));
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2);
  const int vrow = (int)((64 / G::KCH) * vs2 * 2);  // bytes of the rows one instruction covers
  const int lds_k = __builtin_amdgcn_readfirstlane(lds_addr(smem) + hf * G::SLOT + wl * G::LOADS * 1024);
  const int lds_v = lds_k + G::TILE;
  const int lds_wd = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::WORDS + w * 256);

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tc4 = lane & 3;
  const int vrow_l = 4 * (tg >> 1) + tr;
  // V^T fragment (db, ks) and K fragment (kh, t) offsets within a tile, as in
  // the 128-row kernel: the db = 0 / t = 0 offset with 64 db / 32 t XORed in.
  const int vofs0 = vrow_l * (D * 2) + (((2 * (tg & 1) + (tc4 >> 1)) ^ vswz<G::KCH>(vrow_l)) * 16) + (tc4 & 1) * 8;
  const int kofs0 = l32 * (D * 2) + ((half ^ kswz<G::KCH>(l32)) * 16);

  // K tile kt and this wave's 32 row words of the block (info >= 0), else a
  // load past the pool's range (zeros; the launcher bounds the pool so that
  // offset 0xfffffff0 is out of range), so every wave issues LOADS + 1 loads.
  auto issue_k = [&](int kt, int info, bool tile) INLINE {
    const int g0 = kt * kstep;
    if (tile) {
#pragma unroll
      for (int n = 0; n < G::LOADS; ++n) dma16(krs, kgo[n] + g0, lds_k + n * 1024);
    }
    const int off = info >= 0 ? info * (kBlk * 8) + wl * 256 + lane * 4 : (int)0xfffffff0u;
    dma4(irs, off, lds_wd);
  };
  auto issue_v = [&](int kt) INLINE {
    const int g0 = kt * vstep;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) dma16s(vrs, vgo, g0 + n * vrow, lds_v + n * 1024);
  };

  __syncthreads();  // the lists staged
  int kt_cur = 0, info_cur = kBlkSkip;
  // this wave reads the first half's tiles at the current step
  bool sh_cur = hf == 1 && shared_at(0);
  if (cnt > 0) {
    entry(0, kt_cur, info_cur);
    issue_k(kt_cur, info_cur, !sh_cur);
  }
  bf16x8 qf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (row >= 0 && qrow < p.sq) qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
    else qf[t] = bf16x8{};
  }
  wait_all();
  barrier();
  for (int j = 0; j < steps; ++j) {
    const bool act = j < cnt, more = j + 1 < cnt;
    int kt_next = 0, info_next = kBlkSkip;
    if (more) entry(j + 1, kt_next, info_next);
    const bool sh_next = hf == 1 && shared_at(j + 1);
    if (act && !sh_cur) issue_v(kt_cur);
    const char* kb = smem + (sh_cur ? 0 : hf) * G::SLOT;
    const char* vb = kb + G::TILE;

    int kofs = kofs0, vofs = vofs0;
    asm volatile("" : "+v"(kofs), "+v"(vofs));
    const bool ragged = (kt_cur + 1) * BN > p.skv;
    const bool skip = !act || info_cur == kBlkSkip || r0 >= p.sq;
    const bool need_mask = info_cur >= 0 || ragged;
    uint64_t word = ~0ull;  // this lane's row word (bit = visible key)
    if (act && info_cur >= 0) word = *(const uint64_t*)(smem + G::WORDS + w * 256 + l32 * 8);
    if (ragged) word &= (1ull << (p.skv - kt_cur * BN)) - 1ull;

    bf16x8 pf[4];
    if (!skip) {
      f32x16 s[2];
      auto scores = [&]() INLINE {
        s[0] = f32x16{};
        s[1] = f32x16{};
        bf16x8 fr[kQkAhead];
        auto kread = [&](int n) INLINE -> bf16x8 {
          return *(const bf16x8*)(kb + (kofs ^ (32 * (n % KT))) + (n / KT) * 32 * (D * 2));
        };
#pragma unroll
        for (int n = 0; n < kQkAhead; ++n) fr[n] = kread(n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 2 * KT; ++n) {
          const bf16x8 a = fr[n % kQkAhead];
          s[n / KT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[n % KT], s[n / KT], 0, 0, 0);
          if (n + kQkAhead < 2 * KT) fr[n % kQkAhead] = kread(n + kQkAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (need_mask) {
          // this lane's keys 8 (r / 4) + 4 half + r % 4 of each 32-key half
          const uint64_t wsh = word >> (4 * half);
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const uint32_t wk = (uint32_t)(wsh >> (32 * kh));
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!((wk >> (8 * (r >> 2) + (r & 3))) & 1u)) s[kh][r] = -INFINITY;
          }
        }
      };
      float lsum;
      auto probs = [&]() INLINE {
        const float mneg = -m_run * c;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            f32x8 pv;
#pragma unroll
            for (int q = 0; q < 8; ++q)
              pv[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][8 * tp + q], c, mneg));
            pf[kh * 2 + tp] = __builtin_convertvector(pv, bf16x8);
          }
        }
        const bf16x2 one2 = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
        lsum = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2 * q], pf[ks][2 * q + 1]}, one2, lsum, false);
      };
      auto tile_max = [&]() INLINE -> float {
        float mloc = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2)
          mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[0][r], s[0][r + 1]));
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[1][r], s[1][r + 1]));
        return pair_max(mloc);
      };
      // Lazy maximum as in the 128-row kernel: the first tile of the wave
      // starts from its exact maximum; later tiles are redone with theirs
      // only when some lane's share of a row sum leaves [0, 2^32].
      scores();
      if (j == 0) m_run = fmaxf(m_run, tile_max());
      probs();
      if (__any(!(lsum <= kLazyMax))) {
        scores();
        const float m_new = fmaxf(m_run, tile_max());
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        probs();
      }
      l_run += lsum;
    }
    // Every wave has read K(j) and its row words: the next ones may land.
    barrier();
    if (more) issue_k(kt_next, info_next, !sh_next);
    // V(j) landed (K(j + 1) and its row words may still be in flight).
    if (act) {
      if (!more) wait_all();
      else if (sh_next) wait_vmcnt<1>();
      else wait_vmcnt<G::LOADS + 1>();
    }
    barrier();
    if (!skip) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const char* a0 = vb + (vofs ^ (64 * db)) + (16 * ks) * (D * 2);
          bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)a0);
          bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a0 + 8 * (D * 2)));
          bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB - kPvAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kPvAhead, 0);
    }
    // K(j + 1) and its row words landed; every wave is done with V(j).
    wait_all();
    barrier();
    kt_cur = kt_next;
    info_cur = info_next;
    sh_cur = sh_next;
  }
  if (row < 0) return;

  // Epilogue: O = O / l (zero rows for l = 0) staged through LDS (4 KB per
  // wave in its half's K tile, which no wave reads any more) so that every
  // store writes 16-byte pieces of whole 128-byte row segments; LSE in
  // natural log.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  {
    char* stg = smem + hf * G::SLOT + wl * 4096;
    __bf16* Ob = (__bf16*)p.o + it.b * p.os[0] + it.h * p.os[1];
    const int rr = lane >> 3, ch = lane & 7;
#pragma unroll
    for (int rd = 0; rd < D / 64; ++rd) {
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int db = 2 * rd + dh, cc = dh * 4 + rg;
          f32x4 x = f32x4{acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2], acc[db][4 * rg + 3]} * inv;
          *(bf16x4*)(stg + l32 * 128 + ((cc ^ (l32 & 7)) * 16) + half * 8) = __builtin_convertvector(x, bf16x4);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rw = 8 * k + rr;
        const bf16x8 v = *(const bf16x8*)(stg + rw * 128 + ((ch ^ (rw & 7)) * 16));
        if (r0 + rw < p.sq) *(bf16x8*)(Ob + (int64_t)(r0 + rw) * p.os[2] + rd * 64 + ch * 8) = v;
      }
    }
  }
  if (qrow < p.sq && p.lse && half == 0) {
    const float lse = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
    p.lse[((int64_t)it.b * p.hq + it.h) * p.sq + qrow] = lse;
  }
#endif
}

template <int D>
hipError_t launch_d(const TileAttnParams& p, hipStream_t s) {
  const int64_t np = (p.nqt + 1) / 2;
  const int64_t items = (int64_t)p.mb * p.mh * np * p.expand;
  if (items <= 0) return hipSuccess;
  if (items > INT32_MAX / 2) return hipErrorInvalidValue;
  // (K/V head, batch) sets dealt whole to the XCDs when they split evenly,
  // every XCD's share holds all batch masks alike, and one set fills an XCD's
  // workgroup slots (32 CUs x 2)
  const int64_t sets = (int64_t)p.b * p.hkv;
  const int set_major = sets % kXcds == 0 && p.mh == 1 && (p.mb == 1 || (sets / kXcds) % p.b == 0) &&
                        np * p.group >= 64;
  const int gsz = (p.mh == 1) ? p.group : 1;
  const int64_t unit = set_major ? kXcds : (int64_t)kXcds * gsz;
  const int64_t npad = (items + unit - 1) / unit * unit;
  hipLaunchKernelGGL((k_attn_pair<D>), dim3((unsigned)npad), dim3(NT), 0, s, p, (int)items, set_major, gsz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pair_bf16(const TileAttnParams& p, int32_t d, hipStream_t s) {
  if (p.bn != BN || p.bm != HR || p.kind != FMASK_ENC_BITMAP) return hipErrorInvalidValue;
  if (p.pool_cap > ((int64_t)1 << 22)) return hipErrorInvalidValue;  // 32-bit buffer offsets
  if (d == 128) return launch_d<128>(p, s);
  if (d == 64) return launch_d<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
