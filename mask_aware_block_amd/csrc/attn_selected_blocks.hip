// Selected-key attention forward, block-major form (bf16, fp32 accumulation).
//
// Visibility is a per-query list of K/V blocks of 32 cells (llama.cpp
// selected-key PR; the lists arrive canonical: valid, distinct, ascending).
// With many queries the same block sits on the lists of many queries (at 128K
// context, 2048 queries and 64 entries, about 28 queries name each block), so
// walking the lists query by query gathers every block's K and V that many
// times.  This form inverts the lists instead:
//   k_blk_clear, k_blk_hist, k_blk_scan, k_blk_scatter
//       per list batch, the (query, entry) pairs of every block (counting sort
//       by block; the order inside a block does not matter, see below);
//   k_blk_partial   one workgroup per (K/V head, batch, block): the block's K
//       and V go into LDS once; the rows (entry, query head of the group) of
//       the queries that name it are taken 32 at a time per wave, their Q rows
//       gathered into registers, S^T = K Q^T and O^T = V^T P^T on MFMA with the
//       block's exact maximum, and each row's partial state written out: the
//       exp2-domain maximum m, the sum l and O / l in bf16, at the place of its
//       (batch, query, head, entry), with non-temporal stores (read once, by the
//       merge, which loads them non-temporally too);
//   k_blk_combine   one workgroup per (batch, query): per head the partials of
//       its entries merged with factors l_k 2^(m_k - max m) (the split-K rule
//       of the selected-key PR); an empty list gives O = 0 and LSE = -inf.
// Every partial depends only on its own row, and the merge reads them in entry
// order, so the result does not depend on the order the scatter produced.
#include <float.h>

#include "attn_common.h"
#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));  // (m, l) of a partial state

// Direct-to-LDS 16-byte load (as dma16 in device_util.h: M0, one wait state,
// the load) with the non-temporal hint, for data read once: streamed past L2
// rather than evicting what is read again.
__device__ inline void dma16_nt(rsrc_t r, int voff, int lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

constexpr int CELLS = 32;
constexpr int NW = 4;
constexpr int NT = 64 * NW;

// ---------------------------------------------------------------- index

__global__ void __launch_bounds__(256) k_blk_clear(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// hist[mbi][c] += 1 for every valid entry (q, k) of list batch mbi naming block c.
__global__ void __launch_bounds__(256) k_blk_hist(const int32_t* list, const int32_t* count, int mb, int sq,
                                                  int n, int nblk, int32_t* hist) {
  const int64_t total = (int64_t)mb * sq * n;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int k = (int)(i % n);
    const int64_t qi = i / n;  // mbi * sq + q
    if (k < count[qi]) atomicAdd(&hist[(qi / sq) * nblk + list[i]], 1);
  }
}

// off[mbi][0..nblk] = exclusive prefix sums of hist[mbi][*]; one workgroup per
// list batch, 1024 blocks per pass.
__global__ void __launch_bounds__(1024) k_blk_scan(const int32_t* hist, int nblk, int32_t* off) {
  __shared__ int32_t s[1024];
  const int mbi = blockIdx.x, t = threadIdx.x;
  const int32_t* h = hist + (int64_t)mbi * nblk;
  int32_t* o = off + (int64_t)mbi * (nblk + 1);
  int32_t carry = 0;
  for (int base = 0; base < nblk; base += 1024) {
    const int32_t x = base + t < nblk ? h[base + t] : 0;
    s[t] = x;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
      const int32_t y = t >= d ? s[t - d] : 0;
      __syncthreads();
      s[t] += y;
      __syncthreads();
    }
    if (base + t < nblk) o[base + t] = carry + s[t] - x;
    const int32_t tot = s[1023];
    __syncthreads();
    carry += tot;
  }
  if (t == 0) o[nblk] = carry;
}

// inv[mbi][off[c] ..] = (q << 8) | k for the pairs naming block c; hist counts
// back down to zero.
__global__ void __launch_bounds__(256) k_blk_scatter(const int32_t* list, const int32_t* count, int mb, int sq,
                                                     int n, int nblk, const int32_t* off, int32_t* hist,
                                                     int32_t* inv) {
  const int64_t total = (int64_t)mb * sq * n;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int k = (int)(i % n);
    const int64_t qi = i / n;
    if (k >= count[qi]) continue;
    const int64_t mbi = qi / sq;
    const int q = (int)(qi % sq), c = list[i];
    const int pos = off[mbi * (nblk + 1) + c] + atomicSub(&hist[mbi * nblk + c], 1) - 1;
    inv[mbi * (int64_t)sq * n + pos] = (q << 8) | k;
  }
}

// ---------------------------------------------------------------- partials

// Place of the partial state of (batch b, query q, query head h, list entry e)
// in the workspace: the entries of one (query, head) are consecutive, so the
// merge reads each (query, head)'s partial O rows as one contiguous run.
__device__ inline int64_t part_slot(const SelAttnParams& p, int b, int q, int h, int e) {
  return (((int64_t)b * p.sq + q) * p.hq + h) * p.n + e;
}

template <int D>
struct BGeo {
  static constexpr int KCH = D / 8;                  // 16-byte chunks per row
  static constexpr int TILE = CELLS * D * 2;         // one block of K or V
  static constexpr int K0 = 0, V0 = TILE, STG = 2 * TILE;  // staging: 4 KB per wave
  static constexpr int END = STG + NW * 4096;
  static constexpr int LOADS = CELLS * KCH / NT;     // 16-byte loads per lane and tile
  static_assert(CELLS * KCH % NT == 0, "tile must split evenly over the workgroup");
};

// LDS swizzles (XOR on the 16-byte chunk index of a row): K rows by the key's
// low bits (the 32 lanes of a fragment read hit distinct chunks); V rows by
// 4 (key & 3) for the transposing reads (the four rows of a read group and the
// four chunks of each hit distinct bank groups, as with 256-byte rows).
template <int KCH>
__device__ inline int bk_swz(int key) { return key & (KCH - 1); }
__device__ inline int bv_swz(int key) { return 4 * (key & 3); }

// Workgroup item l (K/V-head-major, then batch, then block), the blocks of XCD
// x taking items [x per, (x + 1) per): one K/V head's Q rows (gathered by
// every block of that head) stay in that XCD's L2, while the block's K and V,
// read once, are loaded with the non-temporal hint.
template <int D>
__global__ void __launch_bounds__(NT, 2) k_blk_partial(SelAttnParams p, int nblk, int64_t n_items,
                                                        const int32_t* off, const int32_t* inv, f32x2* pm,
                                                        __bf16* po) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G_ = BGeo<D>;
  constexpr int DB = D / 32;
  constexpr int KT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[G_::END];

  const int64_t per = (n_items + kXcds - 1) / kXcds;
  const int64_t l = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (blockIdx.x / kXcds >= per || l >= n_items) return;
  const int c = (int)(l % nblk);
  const int64_t r = l / nblk;
  const int b = (int)(r % p.b), kvh = (int)(r / p.b);
  const int mbi = p.mb > 1 ? b : 0;
  const int32_t* offm = off + (int64_t)mbi * (nblk + 1);
  const int base = offm[c], cnt = offm[c + 1] - base;
  if (cnt == 0) return;
  const int32_t* entries = inv + (int64_t)mbi * p.sq * p.n + base;
  const int G = p.group;
  const int rows = cnt * G;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];
  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];
  const __bf16* Qb = (const __bf16*)p.q + b * p.qs[0];

  // The block's K and V rows into LDS (range-checked: cells past skv read 0).
  {
    const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
    const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);
    const int lds = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * G_::LOADS * 1024);
    const int key0 = c * CELLS;
#pragma unroll
    for (int i = 0; i < G_::LOADS; ++i) {
      const int P = (w * G_::LOADS + i) * 64 + lane;
      const int key = P / G_::KCH, pc = P % G_::KCH;
      const int ko = (int)((key0 + key) * ks2 * 2 + ((pc ^ bk_swz<G_::KCH>(key)) * 16));
      const int vo = (int)((key0 + key) * vs2 * 2 + ((pc ^ bv_swz(key)) * 16));
      dma16_nt(krs, ko, lds + G_::K0 + i * 1024);
      dma16_nt(vrs, vo, lds + G_::V0 + i * 1024);
    }
  }
  const int valid_keys = min(CELLS, p.skv - c * CELLS);
  const float cs = p.scale * kLog2e;

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tc4 = lane & 3;
  const int vrow_l = 4 * (tg >> 1) + tr;
  const int vofs0 = vrow_l * (D * 2) + (((2 * (tg & 1) + (tc4 >> 1)) ^ bv_swz(vrow_l)) * 16) + (tc4 & 1) * 8;
  const int kofs0 = l32 * (D * 2) + ((half ^ bk_swz<G_::KCH>(l32)) * 16);
  const char* kb = smem + G_::K0;
  const char* vb = smem + G_::V0;
  char* stg = smem + G_::STG + w * 4096;

  // This lane's row of the wave's 32-row tile at t0 (entry e, head g of the
  // group) and its Q row: gathered for the first tile while the block's K and
  // V come in, for each later tile as soon as the previous scores are done.
  bf16x8 qf[KT];
  auto load_q = [&](int t0) INLINE {
    const int row = t0 + l32;
    const bool live = row < rows;
    const int e = live ? row / G : 0, g = row - e * G;
    const int q = entries[e] >> 8;
    const __bf16* src = Qb + (kvh * G + g) * p.qs[1] + (int64_t)q * p.qs[2] + 8 * half;
#pragma unroll
    for (int t = 0; t < KT; ++t) qf[t] = live ? *(const bf16x8*)(src + 16 * t) : bf16x8{};
  };
  if (w * 32 < rows) load_q(w * 32);
  wait_all();
  barrier();

  for (int t0 = w * 32; t0 < rows; t0 += NW * 32) {
    const int row = t0 + l32;
    const bool live = row < rows;
    const int e = live ? row / G : 0, g = row - e * G;
    const int ent = entries[e];
    const int q = ent >> 8;
    const int h = kvh * G + g;

    // S^T = K Q^T: 32 keys x 32 rows, lane = row, keys 8 (r / 4) + 4 half + r % 4
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const bf16x8 a = *(const bf16x8*)(kb + (kofs0 ^ (32 * t)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s, 0, 0, 0);
    }
    if (t0 + NW * 32 < rows) load_q(t0 + NW * 32);  // qf is free once the scores are formed
    if (valid_keys < CELLS) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * half + (i & 3) >= valid_keys) s[i] = -INFINITY;
    }
    float mloc = __builtin_elementwise_maximum(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[i], s[i + 1]));
    const float m2 = pair_max(mloc) * cs;  // the block's exact maximum, exp2 domain
    bf16x8 pf[2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      f32x8 pv;
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * tp + j], cs, -m2));
      pf[tp] = __builtin_convertvector(pv, bf16x8);
    }
    const bf16x2 one2 = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2 * j], pf[ks][2 * j + 1]}, one2, lsum, false);
    const float l_tot = pair_sum(lsum);

    // O^T = V^T P^T, then O / l in bf16 through the wave's staging area:
    // 32 rows x 64 columns at a time, each row written as 128-byte pieces.
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      acc[db] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* a0 = vb + (vofs0 ^ (64 * db)) + (16 * ks) * (D * 2);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)a0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a0 + 8 * (D * 2)));
        bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
      }
    }
    const float inv_l = 1.f / l_tot;  // l >= 1: the maximum's own term
    if (live && half == 0) {
      __builtin_nontemporal_store(f32x2{m2, l_tot}, pm + part_slot(p, b, q, h, ent & 0xff));
    }
    const int rr = lane >> 3, ch = lane & 7;
#pragma unroll
    for (int rd = 0; rd < D / 64; ++rd) {
#pragma unroll
      for (int dh = 0; dh < 2; ++dh) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int db = 2 * rd + dh, cc = dh * 4 + rg;
          f32x4 x = f32x4{acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2], acc[db][4 * rg + 3]} * inv_l;
          *(bf16x4*)(stg + l32 * 128 + ((cc ^ (l32 & 7)) * 16) + half * 8) = __builtin_convertvector(x, bf16x4);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rw = 8 * k + rr, orow = t0 + rw;
        const bf16x8 v = *(const bf16x8*)(stg + rw * 128 + ((ch ^ (rw & 7)) * 16));
        if (orow < rows) {
          const int oe = orow / G, og = orow - oe * G;
          const int oent = entries[oe];
          const int64_t slot = part_slot(p, b, oent >> 8, kvh * G + og, oent & 0xff);
          __builtin_nontemporal_store(v, (bf16x8*)(po + slot * D + rd * 64 + ch * 8));
        }
      }
    }
  }
#endif
}

// ---------------------------------------------------------------- merge

// One workgroup per (batch, query); wave w merges heads w, w + 4, ...  Lane k
// holds entry k's (m, l) (lists have at most 64 entries); each lane then owns
// D / 64 output columns.
template <int D>
__global__ void __launch_bounds__(NT) k_blk_combine(SelAttnParams p, const f32x2* pm, const __bf16* po) {
  constexpr int DPL = D / 64;
  const int64_t bq = blockIdx.x;
  const int b = (int)(bq / p.sq), q = (int)(bq % p.sq);
  const int mbi = p.mb > 1 ? b : 0;
  const int cnt = p.count[(int64_t)mbi * p.sq + q];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __bf16* O = (__bf16*)p.o + b * p.os[0] + (int64_t)q * p.os[2];
  const int64_t slot0 = part_slot(p, b, q, 0, 0);  // + h n + entry
  for (int h = w; h < p.hq; h += NW) {
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    float lse = -INFINITY;
    if (cnt > 0) {
      const f32x2 ml = lane < cnt ? __builtin_nontemporal_load(pm + slot0 + h * p.n + lane)
                                  : f32x2{-FLT_MAX, 0.f};
      float M = ml.x;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
      const float wk = lane < cnt ? ml.y * __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
      float L = wk;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) L += __shfl_xor(L, d);
      const float wn = wk / L;
      const __bf16* src = po + (slot0 + h * p.n) * D + lane * DPL;
      const int64_t stride = D;  // the entries of one (query, head) are consecutive
      int k = 0;
      for (; k + 8 <= cnt; k += 8) {
        typedef __bf16 bfv __attribute__((ext_vector_type(DPL)));
        bfv x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load((const bfv*)(src + (k + u) * stride));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float f = __shfl(wn, k + u);
#pragma unroll
          for (int j = 0; j < DPL; ++j) acc[j] = __builtin_fmaf(f, (float)x[u][j], acc[j]);
        }
      }
      for (; k < cnt; ++k) {
        typedef __bf16 bfv __attribute__((ext_vector_type(DPL)));
        const bfv x = __builtin_nontemporal_load((const bfv*)(src + k * stride));
        const float f = __shfl(wn, k);
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] = __builtin_fmaf(f, (float)x[j], acc[j]);
      }
      lse = (M + __log2f(L)) * 0.6931471805599453f;
    }
    typedef __bf16 bfv __attribute__((ext_vector_type(DPL)));
    bfv out;
#pragma unroll
    for (int j = 0; j < DPL; ++j) out[j] = (__bf16)acc[j];
    *(bfv*)(O + h * p.os[1] + lane * DPL) = out;
    if (p.lse && lane == 0) p.lse[((int64_t)b * p.hq + h) * p.sq + q] = lse;
  }
}

}  // namespace

// Workspace layout of the block-major form (16-byte aligned pieces).
BlkLayout selected_blocks_layout(const SelAttnParams& p, int32_t d) {
  BlkLayout L;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  L.nblk = (p.skv + CELLS - 1) / CELLS;
  size_t o = 0;
  L.hist = o; o += up((size_t)p.mb * L.nblk * 4);
  L.off = o; o += up((size_t)p.mb * (L.nblk + 1) * 4);
  L.inv = o; o += up((size_t)p.mb * p.sq * p.n * 4);
  L.pm = o; o += up((size_t)p.b * p.sq * p.n * p.hq * 8);
  L.po = o; o += up((size_t)p.b * p.sq * p.n * p.hq * d * 2);
  L.total = o;
  return L;
}

hipError_t launch_attn_selected_blocks_bf16(const SelAttnParams& p, int32_t d, void* ws, hipStream_t s) {
  if (p.sq <= 0) return hipSuccess;
  if (d != 128 && d != 256) return hipErrorInvalidValue;
  const BlkLayout L = selected_blocks_layout(p, d);
  char* base = (char*)ws;
  int32_t* hist = (int32_t*)(base + L.hist);
  int32_t* off = (int32_t*)(base + L.off);
  int32_t* inv = (int32_t*)(base + L.inv);
  f32x2* pm = (f32x2*)(base + L.pm);
  __bf16* po = (__bf16*)(base + L.po);
  const int64_t nh = (int64_t)p.mb * L.nblk;
  const int64_t ne = (int64_t)p.mb * p.sq * p.n;
  auto grid = [](int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65535 * 4); };
  if (nh > 0) hipLaunchKernelGGL(k_blk_clear, dim3(grid(nh)), dim3(256), 0, s, hist, nh);
  hipLaunchKernelGGL(k_blk_hist, dim3(grid(ne)), dim3(256), 0, s, p.list, p.count, p.mb, p.sq, p.n, L.nblk, hist);
  hipLaunchKernelGGL(k_blk_scan, dim3((unsigned)p.mb), dim3(1024), 0, s, hist, L.nblk, off);
  hipLaunchKernelGGL(k_blk_scatter, dim3(grid(ne)), dim3(256), 0, s, p.list, p.count, p.mb, p.sq, p.n, L.nblk,
                     off, hist, inv);
  const int64_t items = (int64_t)p.hkv * p.b * L.nblk;  // 0 without keys: every list is empty
  const int64_t per = (items + kXcds - 1) / kXcds;
  if (items > 0 && d == 256)
    hipLaunchKernelGGL((k_blk_partial<256>), dim3((unsigned)(per * kXcds)), dim3(NT), 0, s, p, L.nblk, items, off,
                       inv, pm, po);
  else if (items > 0)
    hipLaunchKernelGGL((k_blk_partial<128>), dim3((unsigned)(per * kXcds)), dim3(NT), 0, s, p, L.nblk, items, off,
                       inv, pm, po);
  const unsigned nbq = (unsigned)((int64_t)p.b * p.sq);
  if (d == 256) hipLaunchKernelGGL((k_blk_combine<256>), dim3(nbq), dim3(NT), 0, s, p, pm, po);
  else hipLaunchKernelGGL((k_blk_combine<128>), dim3(nbq), dim3(NT), 0, s, p, pm, po);
  return hipGetLastError();
}

}  // namespace fmask
