// Masked attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA:
// 128-row query tiles of four 32-row waves, interval or 64 x 64 bitmap
// encoding, three workgroups per CU (three waves per SIMD).
//
// Same arithmetic and register layout as the 128-row kernel of
// attn_bf16.hip (S^T = K Q^T per wave with one query row per lane, online
// softmax in the exp2 domain with a lazy running max, O^T += V^T P^T through
// the transposing LDS read); the difference is the memory plan, which trades
// double-buffered V for occupancy.  LDS per workgroup is 52 KB:
//   K tiles     2 x 16 KB   tile i + 1 streams in while tile i is computed
//   V tile      1 x 16 KB   V(i) streams in behind QK(i) and the softmax
//   mask data   2 x  1 KB   intervals: raw [4][64] int32, one field per wave;
//                           bitmap: each wave's 32 row words of its block
//   per-wave    1 KB        intervals: row masks of PARTIAL tiles;
//                           bitmap: both 64-row blocks of the first 128 list
//                           entries (pool index, or FULL / SKIP)
//   tile list       1 KB
// so three workgroups (12 waves) share a CU, and the MFMA work of one wave
// overlaps the VALU work and load waits of the others.  Per tile:
//   issue V(i), K(i+1), intervals(i+1)   (direct-to-LDS buffer loads)
//   wave state of tile i (SKIP / FULL / PARTIAL for its 32 rows); QK; mask; softmax
//   wait V(i); barrier; PV(i)
//   wait for everything; barrier
// and at the end O goes out through LDS (whole 128-byte row pieces per store).
#include <float.h>

#include "attn_common.h"
#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

constexpr int BN = 64;
constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int BM = 32 * NW;
constexpr int kList = 256;  // tile-list entries staged in LDS
constexpr int kBinfo = 128;  // bitmap: list entries whose block info is staged in LDS

template <int D>
struct Geo {
  static constexpr int KCH = D / 8;
  static constexpr int TILE = BN * D * 2;
  static constexpr int K0 = 0;               // K buffers 0, 1
  static constexpr int V0 = 2 * TILE;        // V buffer
  static constexpr int IV0 = 3 * TILE;       // raw interval buffers 0, 1: [4][BN] int32
  static constexpr int IVB = 4 * BN * 4;
  static constexpr int RM0 = IV0 + 2 * IVB;  // row masks [NW][BN] uint32, or block info [2][kBinfo] int32
  static constexpr int END = RM0 + NW * BN * 4;
  static_assert(2 * kBinfo <= NW * BN, "block info fits the row-mask region");
  static constexpr int LOADS = BN * KCH / NT;
  static_assert(BN * KCH % NT == 0, "tile must split evenly over the workgroup");
};

struct Item {
  int b, h, kvh, mb, mh, qt, row;
};

__device__ inline Item decode_item(const TileAttnParams& p, int l) {
  Item it;
  int r = p.order[l / p.expand];
  int e = l % p.expand;
  it.row = r;
  it.qt = r % p.nqt;
  it.mh = (r / p.nqt) % p.mh;
  it.mb = r / (p.nqt * p.mh);
  if (p.mb == 1 && p.mh == 1) { it.b = e / p.hq; it.h = e % p.hq; }
  else if (p.mb == 1) { it.b = e; it.h = it.mh; }
  else if (p.mh == 1) { it.b = it.mb; it.h = e; }
  else { it.b = it.mb; it.h = it.mh; }
  it.kvh = it.h / p.group;
  return it;
}

// XCD-aware remap: groups of `gsz` consecutive logical items land on one XCD
// while the longest-first order is kept across XCDs.
__device__ inline int logical_item(int gsz) {
  int p = blockIdx.x;
  int xcd = p % kXcds, k = p / kXcds;
  return ((k / gsz) * kXcds + xcd) * gsz + (k % gsz);
}

// Set-major items: item l = ((kvh * b + batch) * nqt + t) * group + j is head
// kvh * group + j of `batch` on the t-th longest tile row of its mask slice.
// The blocks of XCD x (x = blockIdx % 8) take items [x n / 8, (x + 1) n / 8)
// in turn, so an XCD works through whole (K/V head, batch) sets one after
// another: the workgroups on one XCD at a time share one set's K and V, and
// as each walks its keys in ascending order they reuse each other's tiles in
// that XCD's L2.  (The round-robin deal of decode_item spreads every set over
// all XCDs, so each XCD holds several sets' K and V at once.)
__device__ inline Item set_item(const TileAttnParams& p, int l) {
  Item it;
  const int j = l % p.group;
  int r = l / p.group;
  const int t = r % p.nqt;
  r /= p.nqt;
  it.b = r % p.b;
  it.kvh = r / p.b;
  it.h = it.kvh * p.group + j;
  it.mb = p.mb > 1 ? it.b : 0;
  it.mh = p.mh > 1 ? it.h : 0;
  it.row = p.order[(it.mb * p.mh + it.mh) * p.nqt + t];
  it.qt = it.row % p.nqt;
  return it;
}

template <int D, int KIND>
__global__ void __launch_bounds__(NT, 3) k_attn_o3(TileAttnParams p, int gsz) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = Geo<D>;
  constexpr int DB = D / 32;
  constexpr int KT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[G::END];
  __shared__ int32_t lst[kList];

  Item it;
  if (p.set_major) {
    const int per = p.n_items / kXcds, k = blockIdx.x / kXcds;
    if (k >= per) return;
    it = set_item(p, (int)(blockIdx.x % kXcds) * per + k);
  } else {
    const int l = logical_item(gsz);
    if (l >= p.n_items) return;
    it = decode_item(p, l);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int r0 = it.qt * BM + w * 32;  // first row of this wave
  const int qrow = r0 + l32;

  const __bf16* Q = (const __bf16*)p.q + it.b * p.qs[0] + it.h * p.qs[1];
  const __bf16* K = (const __bf16*)p.k + it.b * p.ks[0] + it.kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + it.b * p.vs[0] + it.kvh * p.vs[1];
  const int32_t* list = p.list + (int64_t)it.row * p.nkt;
  const int cnt = p.count[it.row];
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];
  const int32_t* ivcol = p.iv + ((size_t)it.mb * p.mh + it.mh) * 4 * (size_t)p.skv;

  // (LDS is not cleared: every byte a wave reads is written first, K and V
  // tiles entirely by their loads, zeros past the end included)
  for (int i = tid; i < min(cnt, kList); i += NT) lst[i] = list[i];
  auto entry = [&](int i) INLINE -> int {
    return i < kList ? __builtin_amdgcn_readfirstlane(lst[i]) : sload_wait(list + i);
  };
  // Bitmap: the two 64-row blocks (block rows 2 qt and 2 qt + 1) of list entry
  // e; waves 0, 1 use the first, waves 2, 3 the second.
  const size_t bbase = ((size_t)it.mb * p.mh + it.mh) * p.nbq;
  auto block_info = [&](int e, int half_row) INLINE -> int {
    const int bi = 2 * it.qt + half_row, kt = e & 0x7fffffff;
    if (bi >= p.nbq) return kBlkSkip;
    const size_t bx = (bbase + bi) * p.nbk + kt;
    const int st = p.bstate[bx];
    return st == FMASK_PARTIAL ? p.bindex[bx] : (st == FMASK_FULL ? kBlkFull : kBlkSkip);
  };
  int32_t* binfo = (int32_t*)(smem + G::RM0);  // [2][kBinfo]
  if (KIND == FMASK_ENC_BITMAP) {
    for (int i = tid; i < min(cnt, kBinfo); i += NT) {
      const int e = list[i];
      binfo[i] = block_info(e, 0);
      binfo[kBinfo + i] = block_info(e, 1);
    }
  }
  // This wave's block of list entry i (entry value e).  Past the staged
  // entries the block is read with scalar loads: a vector load's wait would
  // also drain the tile loads in flight.
  const int qt_u = __builtin_amdgcn_readfirstlane(it.qt);
  const int64_t bbase_u = (int64_t)__builtin_amdgcn_readfirstlane((int)(bbase));
  auto wave_block = [&](int i, int e) INLINE -> int {
    if (i < kBinfo) return __builtin_amdgcn_readfirstlane(binfo[(w >> 1) * kBinfo + i]);
    const int bi = 2 * qt_u + (w >> 1), kt = e & 0x7fffffff;
    if (bi >= p.nbq) return kBlkSkip;
    const int64_t bx = (bbase_u + bi) * p.nbk + kt;
    const int st = sload_byte(p.bstate + bx);
    return st == FMASK_PARTIAL ? sload_wait(p.bindex + bx) : (st == FMASK_FULL ? kBlkFull : kBlkSkip);
  };


  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = p.scale * kLog2e;

  const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);
  const rsrc_t irs = KIND == FMASK_ENC_BITMAP ? make_rsrc(p.bbits, p.pool_cap * kBlk * 8)
                                              : make_rsrc(ivcol, (int64_t)4 * p.skv * 4);
  // Direct-to-LDS loads: instruction n of wave w fills LDS chunks
  // P = (w * LOADS + n) * 64 + lane, i.e. row P / KCH, physical chunk P % KCH
  // holding logical chunk (P % KCH) ^ swizzle(row).
  // The V swizzle does not depend on n (rows advance by a multiple of 4 per
  // instruction), so one lane offset serves all of V's loads; the rest is a
  // scalar offset.
  int kgo[G::LOADS];
#pragma unroll
  for (int n = 0; n < G::LOADS; ++n) {
    const int P = (w * G::LOADS + n) * 64 + lane;
    const int key = P / G::KCH, pc = P % G::KCH;
    kgo[n] = (int)(key * ks2 * 2 + ((pc ^ kswz<G::KCH>(key)) * 16));
  }
  int vgo;
  {
    const int P = w * G::LOADS * 64 + lane;
    const int key = P / G::KCH, pc = P % G::KCH;
    vgo = (int)(key * vs2 * 2 + ((pc ^ vswz<G::KCH>(key)) * 16));
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2);
  const int vrow = (int)((64 / G::KCH) * vs2 * 2);  // bytes of the rows one instruction covers
  const int lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * G::LOADS * 1024);
  const int lds_iv = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::IV0 + w * BN * 4);

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tc4 = lane & 3;
  const int vrow_l = 4 * (tg >> 1) + tr;
  // V^T fragment (db, ks): chunk 4 db + x of row vrow_l + 16 ks, i.e. the
  // db = 0 offset with 64 db XORed into the swizzled chunk bits.  K fragment
  // (kh, t): chunk 2 t + half of key kh * 32 + l32, i.e. the t = 0 offset with
  // 32 t XORed in (the swizzle only touches the chunk bits).
  const int vofs0 = vrow_l * (D * 2) + (((2 * (tg & 1) + (tc4 >> 1)) ^ vswz<G::KCH>(vrow_l)) * 16) + (tc4 & 1) * 8;
  const int kofs0 = l32 * (D * 2) + ((half ^ kswz<G::KCH>(l32)) * 16);

  // K tile kt (list entry i, value e) and its mask data: LOADS + 1 loads.
  // Intervals: wave w loads field w.  Bitmap: wave w loads the 32 words of its
  // rows when its block is PARTIAL, else a load past the pool's range (zeros)
  // so that every wave always issues the same number of loads.  The pool's
  // buffer resource spans pool_cap * 512 bytes <= 2^31 (the launcher refuses
  // larger pools: buffer offsets and num_records are 32-bit), so the dummy
  // offset 0xfffffff0 is out of range for every accepted pool.
  auto issue_k = [&](int i, int e, int buf) INLINE {
    const int kt = e & 0x7fffffff;
    const int base = lds_w + G::K0 + buf * G::TILE, g0 = kt * kstep;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) dma16(krs, kgo[n] + g0, base + n * 1024);
    if (KIND == FMASK_ENC_BITMAP) {
      const int info = wave_block(i, e);
      const int off = info >= 0 ? info * (kBlk * 8) + (w & 1) * 256 + lane * 4 : (int)0xfffffff0u;
      dma4(irs, off, lds_iv + buf * G::IVB);
    } else {
      dma4(irs, (w * p.skv + kt * BN + lane) * 4, lds_iv + buf * G::IVB);
    }
  };
  // V tile kt: LOADS loads.
  auto issue_v = [&](int kt) INLINE {
    const int base = lds_w + G::V0, g0 = kt * vstep;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) dma16s(vrs, vgo, g0 + n * vrow, base + n * 1024);
  };

  __syncthreads();  // the list (and block info) staged
  // The first K tile's loads fly while Q comes in.  (Every wait on the
  // vector-memory counter drains the oldest loads first, so the compiler's
  // waits for Q, which know nothing of the tile loads, still cover Q.)
  const int e0 = cnt > 0 ? entry(0) : 0;
  if (cnt > 0) issue_k(0, e0, 0);
  bf16x8 qf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (qrow < p.sq) qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
    else qf[t] = bf16x8{};
  }
  if (cnt > 0) {
    int e_cur = e0;
    wait_all();
    barrier();
    for (int i = 0; i < cnt; ++i) {
      const bool more = i + 1 < cnt;
      const int b = i & 1;
      const int kt = e_cur & 0x7fffffff;
      const int e_next = more ? entry(i + 1) : 0;
      issue_v(kt);
      if (more) issue_k(i + 1, e_next, b ^ 1);

      // (laundered so that the XORed offsets are formed where they are used
      // rather than held in registers across the loop)
      int kofs = kofs0 + b * G::TILE, vofs = vofs0;
      asm volatile("" : "+v"(kofs), "+v"(vofs));
      const char* kb = smem + G::K0;
      const char* vb = smem + G::V0;
      const int32_t* raw = (const int32_t*)(smem + G::IV0 + b * G::IVB);
      const bool ragged = (kt + 1) * BN > p.skv;
      bool need_mask = !(e_cur & (int)FMASK_LIST_FULL_BIT) || ragged;
      bool skip = false;
      uint32_t* rmask = (uint32_t*)(smem + G::RM0) + w * BN;
      uint64_t word = ~0ull;  // bitmap: this lane's row word (bit = visible key)
      if (KIND == FMASK_ENC_BITMAP) {
        const int info = wave_block(i, e_cur);
        skip = info == kBlkSkip || r0 >= p.sq;
        need_mask = info >= 0 || ragged;
        if (info >= 0) word = *(const uint64_t*)(smem + G::IV0 + b * G::IVB + w * 256 + l32 * 8);
        if (ragged) word &= (1ull << (p.skv - kt * BN)) - 1ull;
      } else if (need_mask) {
        // This wave's 32-bit row mask of each key column (lane = key; bit r set
        // iff row r0 + r is masked; keys past skv are masked for every row),
        // and from it the wave's state for the tile.
        const int key = kt * BN + lane;
        int us = raw[lane], ue = raw[BN + lane], ls = raw[2 * BN + lane], le = raw[3 * BN + lane];
        if (key >= p.skv) { us = 0; ue = 0x7fffffff; ls = 0; le = 0; }
        auto bits = [&](int a, int e) INLINE -> uint32_t {
          const int lo = min(max(a - r0, 0), 32), hi = min(max(e - r0, 0), 32);
          return (uint32_t)(((1ull << hi) - 1ull) & ~((1ull << lo) - 1ull));
        };
        const uint32_t mk = bits(us, ue) | bits(ls, le);
        rmask[lane] = mk;
        const int n = min(max(p.sq - r0, 0), 32);
        const uint32_t valid = (uint32_t)((1ull << n) - 1ull);
        skip = __ballot((mk & valid) == valid) == ~0ull;
        need_mask = __ballot((mk & valid) != 0u) != 0ull;
      }

      bf16x8 pf[4];
      if (!skip) {
        // S^T = K Q^T for the two 32-key halves: 2 D / 16 MFMAs, each K
        // fragment read kQkAhead MFMAs ahead into a ring of registers
        // (sched_barrier keeps the scheduler from sinking the reads back next
        // to their MFMAs); then the tile's mask.
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
            // bitmap: this lane's keys 8 (r / 4) + 4 half + r % 4 of each half,
            // shifted so that the bit positions are constants
            const uint64_t wl = word >> (4 * half);
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
              const uint32_t wk = (uint32_t)(wl >> (32 * kh));
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int kl = kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (KIND == FMASK_ENC_BITMAP) {
                  if (!((wk >> (8 * (r >> 2) + (r & 3))) & 1u)) s[kh][r] = -INFINITY;
                } else {
                  if ((rmask[kl] >> l32) & 1u) s[kh][r] = -INFINITY;
                }
              }
            }
          }
        };
        // P = exp2(S c - m c) in bf16 against the running maximum m, and this
        // lane's share of the row sum.
        float lsum;
        auto probs = [&]() INLINE {
          const float mneg = -m_run * c;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
              f32x8 pv;
#pragma unroll
              for (int j = 0; j < 8; ++j)
                pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][8 * tp + j], c, mneg));
              pf[kh * 2 + tp] = __builtin_convertvector(pv, bf16x8);
            }
          }
          const bf16x2 one2 = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
          lsum = 0.f;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2 * j], pf[ks][2 * j + 1]}, one2, lsum, false);
        };
        // Online softmax with a lazy maximum: the tile's probabilities are
        // formed against the running maximum without taking the tile's own
        // maximum first.  Only when some lane's share of a row sum leaves
        // [0, 2^kLazyLog2] (a row's first visible tile when that is not the
        // wave's first tile, so that the running maximum is still -FLT_MAX and
        // P overflows, or scores that grew by more than kLazyLog2 in the exp2
        // domain) is the tile redone with its exact
        // maximum: S again (K is still staged), the maximum over both key halves
        // (IEEE maximum, the other 32 keys of a row sit in lane ^ 32), O and l
        // rescaled, P again.  In between P may exceed 1 by up to 2^kLazyLog2,
        // which bf16 and the fp32 sums carry without loss of relative precision.
        scores();
        if (i == 0) {
          // first tile of the row: start from its exact maximum (O and l are
          // still zero), so that the lazy attempt below holds
          float mloc = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
          for (int r = 2; r < 16; r += 2)
            mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[0][r], s[0][r + 1]));
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[1][r], s[1][r + 1]));
          m_run = fmaxf(m_run, pair_max(mloc));
        }
        probs();
        if (__any(!(lsum <= kLazyMax))) {
          scores();
          float mloc = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
          for (int r = 2; r < 16; r += 2)
            mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[0][r], s[0][r + 1]));
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[1][r], s[1][r + 1]));
          const float m_new = fmaxf(m_run, pair_max(mloc));
          const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] *= alpha;
          probs();
        }
        l_run += lsum;
      }
      // V(i) landed (K(i+1) and its intervals may still be in flight).
      if (more) wait_vmcnt<G::LOADS + 1>();
      else wait_all();
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
        // Same for the V^T fragments (two transposing reads per MFMA).
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvAhead, 0);
#pragma unroll
        for (int i = 0; i < 4 * DB - kPvAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kPvAhead, 0);
      }
      // K(i+1) and its intervals landed; every wave is done with V(i) and K(i).
      wait_all();
      barrier();
      e_cur = e_next;
    }
  }

  // Epilogue: O = O / l (zero rows for l = 0), staged through LDS so that
  // every store writes 16-byte pieces of whole 128-byte row segments; LSE in
  // natural log.  Each wave stages 32 rows x 64 columns at a time in its own
  // 4 KB of the K buffers, which no wave reads any more.
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  {
    char* stg = smem + G::K0 + w * 4096;
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
        const int row = 8 * k + rr;
        const bf16x8 v = *(const bf16x8*)(stg + row * 128 + ((ch ^ (row & 7)) * 16));
        if (r0 + row < p.sq) *(bf16x8*)(Ob + (int64_t)(r0 + row) * p.os[2] + rd * 64 + ch * 8) = v;
      }
    }
  }
  if (qrow < p.sq && p.lse && half == 0) {
    const float lse = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
    p.lse[((int64_t)it.b * p.hq + it.h) * p.sq + qrow] = lse;
  }
#endif
}

template <int D, int KIND>
hipError_t launch_d(const TileAttnParams& p, hipStream_t s) {
  const int gsz = (p.mh == 1) ? p.group : 1;
  if (p.n_items <= 0) return hipSuccess;
  const int64_t unit = p.set_major ? kXcds : (int64_t)kXcds * gsz;
  const int64_t npad = (p.n_items + unit - 1) / unit * unit;
  hipLaunchKernelGGL((k_attn_o3<D, KIND>), dim3((unsigned)npad), dim3(NT), 0, s, p, gsz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_o3_bf16(const TileAttnParams& p, int32_t d, hipStream_t s) {
  if (p.bn != BN || p.bm != BM) return hipErrorInvalidValue;
  if (p.kind == FMASK_ENC_INTERVALS) {
    if (d == 128) return launch_d<128, FMASK_ENC_INTERVALS>(p, s);
    if (d == 64) return launch_d<64, FMASK_ENC_INTERVALS>(p, s);
  } else if (p.kind == FMASK_ENC_BITMAP) {
    if (p.pool_cap > ((int64_t)1 << 22)) return hipErrorInvalidValue;  // 32-bit buffer offsets
    if (d == 128) return launch_d<128, FMASK_ENC_BITMAP>(p, s);
    if (d == 64) return launch_d<64, FMASK_ENC_BITMAP>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fmask
