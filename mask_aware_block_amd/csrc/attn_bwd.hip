// Backward pass of the masked attention forward, bf16 inputs, fp32
// accumulation, gfx950 MFMA (interval and 64 x 64 bitmap encodings, 128 x 64
// tile table).
//
// With P_ij = exp(s_ij - LSE_i) on visible cells, D_i = sum_d dO_id O_id and
// dS = P * (dO V^T - D):  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Two launches, no atomics:
//   k_bwd_dq     one 128-row query tile per workgroup (four 32-row waves)
//                walking the tile row's compact list of 64-key tiles, as in
//                the forward: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, then
//                dQ^T += K^T dS^T.  Its prologue forms each row's D_i (from
//                the row's dO, already in registers, and O) and LSE_i log2(e)
//                (+inf for rows with no visible key, so that their P is
//                exactly 0), and leaves both in the workspace for the dK/dV
//                kernel, which runs after it.
//   k_bwd_dkdv   one 64-key tile per workgroup walking its column list of
//                128-row query tiles, for every query head of the K/V head:
//                S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//                dK^T += Q^T dS.  Query tiles are double-buffered in LDS.
//                D = 64: four waves split the keys (2 x 32) and the rows of
//                each query tile (2 x 64), with K and V in registers; the two
//                row halves are summed through LDS at the end.
//   k_bwd_dkdv8  the D = 128 form: eight waves (2 x 32 keys, 4 x 32 rows),
//                two per SIMD, with K in registers and V staged in LDS; the
//                four row quarters are summed through LDS in two rounds.
// Tiles whose rows and keys a wave does not see at all are skipped per wave;
// FULL tiles run without element masks.  With a bitmap mask each wave's rows
// lie in one 64 x 64 block of the key tile: the dQ kernel masks with its row's
// word of the block (bit = key), the dK/dV kernel with its key's column of the
// block, gathered from the row words by one ballot per key.  Operand fragments that are read
// both row-wise (16-byte reads) and transposed (ds_read_b64_tr_b16) live in
// LDS under a swizzle that keeps both access patterns free of bank conflicts,
// and every MFMA operand read from LDS is read kAhead MFMAs ahead into a ring
// of registers (the four-wave dK/dV kernel runs one wave per SIMD, so nothing
// else hides the LDS latency).  The file is compiled with VGPR-form MFMAs (build.py).
#include <float.h>

#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS FMASK_LDS_AS
#define INLINE __attribute__((always_inline))

constexpr int BN = 64;    // keys per tile
constexpr int BM = 128;   // query rows per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAhead = 3;  // operand fragments read ahead of their MFMA

// 16-byte chunk swizzle serving both access patterns: 16 consecutive rows
// read at one logical chunk hit 16 distinct (bank) positions, and the four
// rows of a transposing read group hit distinct chunk pairs.
template <int KCH>
__device__ inline int sw(int row) {
  if (KCH == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 3) << 1) | ((row >> 3) & 1);  // KCH == 8
}

// Byte offset (inside a [rows][D] bf16 tile) of logical chunk ch of row r.
template <int D>
__device__ inline int chunk_off(int r, int ch) {
  return r * (D * 2) + ((ch ^ sw<D / 8>(r)) * 16);
}

// Transposing-read offsets: lane (g = lane / 16, rr = (lane % 16) / 4,
// c4 = lane % 4) addresses row 4 (g / 2) + rr and the 8 bytes at
// d = 32 db + 16 (g % 2) + 4 c4 of a group of 16 rows; the read hands lane l
// four rows at d = 32 db + (l % 32), which become the MFMA operand slots
// 8 (j / 4) + 4 (l / 32) + j % 4 of a 16-row step (the slot order the score
// accumulators produce).
// (hi selects rows 8 .. 15 of the group.)
template <int D>
__device__ inline int tr_off(int lane, int db, int hi) {
  const int tg = lane >> 4, rr = (lane >> 2) & 3, tc4 = lane & 3;
  const int row = 8 * hi + 4 * (tg >> 1) + rr;
  const int ch = 4 * db + 2 * (tg & 1) + (tc4 >> 1);
  return chunk_off<D>(row, ch) + (tc4 & 1) * 8;
}

// A 32 x 16 operand fragment (32 values of d, k = 16 rows of the tile) read
// transposed from a swizzled [rows][D] tile, rows r0 .. r0 + 15 (r0 % 16 == 0;
// the swizzle depends on row % 16 only, so the offsets of rows 0 .. 15 serve).
template <int D>
__device__ inline bf16x8 tr_frag(const char* tile, int r0, int off_lo, int off_hi) {
  const char* t = tile + r0 * (D * 2);
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(t + off_lo));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(t + off_hi));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline int overlap(int a0, int a1, int b0, int b1) {
  return max(0, min(a1, b1) - max(a0, b0));
}

__device__ inline int logical_item(int gsz) {
  int p = blockIdx.x;
  int xcd = p % kXcds, k = p / kXcds;
  return ((k / gsz) * kXcds + xcd) * gsz + (k % gsz);
}

// ------------------------------------------------------------------ dQ
template <int D>
struct GeoQ {
  static constexpr int KCH = D / 8;
  static constexpr int TILE = BN * D * 2;
  static constexpr int STAGE = 2 * TILE + 4 * BN * 4;  // K, V, raw intervals [4][BN]
  static constexpr int RM0 = 2 * STAGE;                // per-wave row masks [4][BN]
  static constexpr int END = RM0 + 4 * BN * 4;
  static constexpr int LOADS = BN * KCH / 256;
};

template <int D, int KIND>
__global__ void __launch_bounds__(256, 2) k_bwd_dq(BwdParams p, int expand, int n_items, int gsz) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = GeoQ<D>;
  constexpr int DB = D / 32, KT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[G::END];

  const int l = logical_item(gsz);
  if (l >= n_items) return;
  // item -> (mask row, batch, head), as the forward orders them
  // (the row uniform, so that its list entries are read with scalar loads)
  const int row = __builtin_amdgcn_readfirstlane(p.order[l / expand]), e = l % expand;
  const int qt = row % p.nqt, mh = (row / p.nqt) % p.mh, mb = row / (p.nqt * p.mh);
  int b, h;
  if (p.mb == 1 && p.mh == 1) { b = e / p.hq; h = e % p.hq; }
  else if (p.mb == 1) { b = e; h = mh; }
  else if (p.mh == 1) { b = mb; h = e; }
  else { b = mb; h = mh; }
  const int kvh = h / p.group;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int r0 = qt * BM + w * 32;
  const int qrow = r0 + l32;
  const int32_t* list = p.list + (int64_t)row * p.nkt;
  const int cnt = sload_wait(p.count + row);
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];
  const int32_t* ivcol = KIND == FMASK_ENC_BITMAP ? p.iv : p.iv + ((size_t)mb * p.mh + mh) * 4 * (size_t)p.skv;
  const __bf16* Q = (const __bf16*)p.q + b * p.qs[0] + h * p.qs[1];
  const __bf16* dO = (const __bf16*)p.dout + b * p.os[0] + h * p.os[1];
  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];

  for (int i = tid; i < G::END / 16; i += 256) ((i32x4*)smem)[i] = i32x4{0, 0, 0, 0};

  // Q^T and dO^T as MFMA B operands (lane: row qrow, d = 16 t + 8 half + 0..7)
  bf16x8 qf[KT], df[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (qrow < p.sq) {
      qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
      df[t] = *(const bf16x8*)(dO + qrow * p.os[2] + 16 * t + 8 * half);
    } else {
      qf[t] = bf16x8{};
      df[t] = bf16x8{};
    }
  }
  // D_i = sum_d dO_id O_id: this lane's half of row qrow (the d of its dO
  // fragments), then the other half from lane ^ 32; with LSE_i log2(e) it goes
  // to the workspace for the dK/dV kernel (every row of every (batch, query
  // head) belongs to exactly one item of this launch).
  float dpart = 0.f, lse2 = INFINITY;
  const int64_t g = ((int64_t)b * p.hq + h) * p.sq + qrow;
  if (qrow < p.sq) {
    const __bf16* Orow = (const __bf16*)p.o + b * p.os[0] + h * p.os[1] + qrow * p.os[2] + 8 * half;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const bf16x8 x = *(const bf16x8*)(Orow + 16 * t);
#pragma unroll
      for (int j = 0; j < 8; ++j) dpart += (float)x[j] * (float)df[t][j];
    }
    const float lse = p.lse[g];
    lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
  }
  const float dlt = dpart + __shfl_xor(dpart, 32);
  if (qrow < p.sq && half == 0) {
    p.ws[2 * g] = dlt;
    p.ws[2 * g + 1] = lse2;
  }
  wait_all();  // nothing tracked may stay pending once untracked loads fly

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
  const float c = p.scale * kLog2e;

  const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);
  const rsrc_t irs = make_rsrc(ivcol, (int64_t)4 * p.skv * 4);
  int kgo[G::LOADS], vgo[G::LOADS];
#pragma unroll
  for (int n = 0; n < G::LOADS; ++n) {
    const int P = (w * G::LOADS + n) * 64 + lane;
    const int key = P / G::KCH, pc = P % G::KCH;
    kgo[n] = (int)(key * ks2 * 2 + ((pc ^ sw<G::KCH>(key)) * 16));
    vgo[n] = (int)(key * vs2 * 2 + ((pc ^ sw<G::KCH>(key)) * 16));
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2);
  const int lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * G::LOADS * 1024);
  const int lds_iv = __builtin_amdgcn_readfirstlane(lds_addr(smem) + 2 * G::TILE + w * BN * 4);
  int tlo[DB], thi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tlo[db] = tr_off<D>(lane, db, 0);
    thi[db] = tr_off<D>(lane, db, 1);
  }

  int st_next = FMASK_SKIP;  // bitmap: this wave's block state of the tile last issued
  auto issue = [&](int kt, int buf) INLINE {
    const int base = lds_w + buf * G::STAGE;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) dma16(krs, kgo[n] + kt * kstep, base + n * 1024);
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) dma16(vrs, vgo[n] + kt * vstep, base + G::TILE + n * 1024);
    if constexpr (KIND != FMASK_ENC_BITMAP) {
      dma4(irs, (w * p.skv + kt * BN + lane) * 4, lds_iv + buf * G::STAGE);
    } else {
      // this wave's 64 x 64 block of key tile kt (state read with a scalar
      // load) and, when PARTIAL, the row words of its 32 rows, loaded into this wave's share
      // of the stage's interval area (which the bitmap form does not use)
      const int bi = 2 * qt + (w >> 1);
      int st = FMASK_SKIP;
      if (bi < p.nbq) {
        const int64_t x = ((int64_t)(mb * p.mh + mh) * p.nbq + bi) * p.nbk + kt;
        st = sload_byte(p.bstate + x);
        if (st == FMASK_PARTIAL) {
          const int pool = sload_wait(p.bindex + x);
          dma4(make_rsrc(p.bbits + (int64_t)pool * 64 + (w & 1) * 32, 256), lane * 4, lds_iv + buf * G::STAGE);
        }
      }
      st_next = st;
    }
  };

  uint32_t* rmask = (uint32_t*)(smem + G::RM0) + w * BN;
  __syncthreads();
  if (cnt > 0) {
    // (list entries by scalar loads: they wait on the scalar counter only,
    // never on the vector-memory counter that the tile loads in flight hold up)
    int e_cur = sload_wait(list);
    issue(e_cur & 0x7fffffff, 0);
    int st_cur = st_next;
    wait_all();
    barrier();
    for (int i = 0; i < cnt; ++i) {
      const bool more = i + 1 < cnt;
      const int e_next = more ? sload_wait(list + i + 1) : 0;
      if (more) issue(e_next & 0x7fffffff, (i + 1) & 1);
      const int kt = e_cur & 0x7fffffff;
      const char* kb = smem + (i & 1) * G::STAGE;
      const char* vb = kb + G::TILE;
      const int32_t* raw = (const int32_t*)(kb + 2 * G::TILE);
      const bool ragged = (kt + 1) * BN > p.skv;
      bool need_mask = !(e_cur & (int)FMASK_LIST_FULL_BIT) || ragged;
      bool skip = false;
      // Bitmap: this wave's 32 rows lie in one 64 x 64 block of the key tile;
      // bit c of `vis` says key kt BN + c is visible to this lane's row
      uint64_t vis = ~0ull;
      if constexpr (KIND == FMASK_ENC_BITMAP) {
        const int st = st_cur;
        skip = st == FMASK_SKIP;
        need_mask = !skip && (st == FMASK_PARTIAL || ragged);
        if (need_mask) {
          if (st == FMASK_PARTIAL) vis = *(const uint64_t*)((const char*)raw + w * BN * 4 + l32 * 8);
          const int nk = p.skv - kt * BN;  // keys of this tile below skv
          if (nk < 64) vis &= (1ull << nk) - 1ull;
        }
      } else if (need_mask) {
        const int key = kt * BN + lane;
        int us = raw[lane], ue = raw[BN + lane], ls = raw[2 * BN + lane], le = raw[3 * BN + lane];
        if (key >= p.skv) { us = 0; ue = 0x7fffffff; ls = 0; le = 0; }
        auto bits = [&](int a, int z) INLINE -> uint32_t {
          const int lo = min(max(a - r0, 0), 32), hi = min(max(z - r0, 0), 32);
          return (uint32_t)(((1ull << hi) - 1ull) & ~((1ull << lo) - 1ull));
        };
        const uint32_t mk = bits(us, ue) | bits(ls, le);
        rmask[lane] = mk;
        const int n = min(max(p.sq - r0, 0), 32);
        const uint32_t valid = (uint32_t)((1ull << n) - 1ull);
        skip = __ballot((mk & valid) == valid) == ~0ull;
        need_mask = __ballot((mk & valid) != 0u) != 0ull;
      }
      if (!skip) {
        // S^T = K Q^T and dP^T = V dO^T for the two 32-key halves: MFMA n is
        // key half n / 2 KT, S for n / KT even, dP for odd; its K or V
        // fragment is read kAhead MFMAs ahead into a ring of registers
        f32x16 s[2], dp[2];
        {
          auto frag = [&](int n) INLINE -> bf16x8 {
            const int kh = n / (2 * KT), t = n % KT;
            return *(const bf16x8*)(((n / KT) & 1 ? vb : kb) + chunk_off<D>(kh * 32 + l32, 2 * t + half));
          };
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) s[kh] = dp[kh] = f32x16{};
          bf16x8 fr[kAhead];
#pragma unroll
          for (int n = 0; n < kAhead; ++n) fr[n] = frag(n);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int n = 0; n < 4 * KT; ++n) {
            const int kh = n / (2 * KT), t = n % KT;
            const bf16x8 a = fr[n % kAhead];
            if ((n / KT) & 1) dp[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[t], dp[kh], 0, 0, 0);
            else s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kh], 0, 0, 0);
            if (n + kAhead < 4 * KT) fr[n % kAhead] = frag(n + kAhead);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // P^T and dS^T (key slots in the order the PV-style operand expects)
        bf16x8 dsf[4];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            // bitmap: the keys of this half (32 kh ..), from bit 4 half on
            const uint32_t vw = (uint32_t)(vis >> (32 * kh)) >> (4 * half);
            f32x8 x;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int r = 8 * tp + j;
              const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][r], c, -lse2));
              x[j] = pr * (dp[kh][r] - dlt);
            }
            // element masks of a PARTIAL tile in one pass (one uniform branch,
            // not one per element; a masked value is replaced, whatever it was)
            if (need_mask) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int r = 8 * tp + j;
                const int kl = kh * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if constexpr (KIND == FMASK_ENC_BITMAP) {
                  // all ones where the key is visible: keep the value's bits
                  const int32_t kb = __builtin_amdgcn_sbfe((int32_t)vw, 8 * (r >> 2) + (r & 3), 1);
                  x[j] = __int_as_float(__float_as_int(x[j]) & kb);
                } else {
                  x[j] = ((rmask[kl] >> l32) & 1u) ? 0.f : x[j];
                }
              }
            }
            dsf[kh * 2 + tp] = __builtin_convertvector(x, bf16x8);
          }
        }
        // dQ^T += K^T dS^T (MFMA m: db = m / 4, ks = m % 4; fragments read ahead)
        {
          auto frag = [&](int m) INLINE -> bf16x8 { return tr_frag<D>(kb, 16 * (m % 4), tlo[m / 4], thi[m / 4]); };
          bf16x8 fr[kAhead];
#pragma unroll
          for (int m = 0; m < kAhead; ++m) fr[m] = frag(m);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < 4 * DB; ++m) {
            acc[m / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % kAhead], dsf[m % 4], acc[m / 4], 0, 0, 0);
            if (m + kAhead < 4 * DB) fr[m % kAhead] = frag(m + kAhead);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wait_all();  // tile i+1 landed; every wave is done with tile i
      barrier();
      e_cur = e_next;
      st_cur = st_next;
    }
  }

  if (qrow < p.sq) {
    __bf16* dQ = (__bf16*)p.dq + b * p.qs[0] + h * p.qs[1] + qrow * p.qs[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = db * 32 + 8 * rg + 4 * half;
        f32x4 x = f32x4{acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2], acc[db][4 * rg + 3]} *
                  p.scale;
        *(bf16x4*)(dQ + d0) = __builtin_convertvector(x, bf16x4);
      }
    }
  }
#endif
}

// ------------------------------------------------------------------ dK, dV
template <int D>
struct GeoKV {
  static constexpr int KCH = D / 8;
  static constexpr int TILE = BM * D * 2;        // one [128 rows][D] bf16 tile
  static constexpr int Q0 = 0, DO0 = TILE;       // Q tile, dO tile
  static constexpr int RW0 = 2 * TILE;           // [128 rows] x {D_i, LSE2_i}
  static constexpr int STAGE = RW0 + BM * 8;     // two stages (double-buffered)
  static constexpr int BW0 = 2 * STAGE;          // bitmap: [2 stages][4 waves] x 64 row words
  static constexpr int END = BW0 + 2 * 4 * 512;
  static constexpr int LOADS = BM * KCH / 256;
};

// dK/dV work item l -> (mask column, batch, K/V head).  With one mask for all
// heads the columns come longest first, each expanded over (batch if the mask
// is shared along it) x K/V head; with per-head masks items are (batch, K/V
// head, key tile) in natural order, and the column is that of the head group's
// first head (the kernels walk the group's heads).
__device__ inline void kv_item(const BwdParams& p, int expand, int l, int* col, int* b, int* g) {
  if (p.mh == 1) {
    *col = p.col_order[l / expand];
    const int e = l % expand;
    if (p.mb == 1) { *b = e / p.hkv; *g = e % p.hkv; }
    else { *b = *col / p.nkt; *g = e; }
  } else {
    const int kt0 = l % p.nkt;
    *g = (l / p.nkt) % p.hkv;
    *b = l / (p.nkt * p.hkv);
    *col = ((p.mb == 1 ? 0 : *b) * p.mh) * p.nkt + kt0;
  }
}

template <int D, int KIND>
__global__ void __launch_bounds__(256, 1) k_bwd_dkdv(BwdParams p, int expand, int n_items) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = GeoKV<D>;
  constexpr int DB = D / 32, KT = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[G::END];

  const int l = blockIdx.x;
  if (l >= n_items) return;
  int col, b, g;
  kv_item(p, expand, l, &col, &b, &g);
  // (uniform, so that list and block-state reads below are scalar loads)
  col = __builtin_amdgcn_readfirstlane(col);
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  const int kt = col % p.nkt;
  const int mb = (p.mb == 1) ? 0 : b;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = w & 1, rw = w >> 1;  // key half (32 keys), 64-row half of each query tile
  const int half = lane >> 5, l32 = lane & 31;
  const int key = kt * BN + kw * 32 + l32;  // this lane's key (as MFMA column)

  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + g * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + g * p.vs[1];

  for (int i = tid; i < G::END / 16; i += 256) ((i32x4*)smem)[i] = i32x4{0, 0, 0, 0};
  __syncthreads();  // every wave's clearing stores done before any tile load lands

  // K and V as B operands of S = Q K^T and dP = dO V^T (lane: key, 8 d)
  bf16x8 kf[KT], vf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (key < p.skv) {
      kf[t] = *(const bf16x8*)(K + key * p.ks[2] + 16 * t + 8 * half);
      vf[t] = *(const bf16x8*)(V + key * p.vs[2] + 16 * t + 8 * half);
    } else {
      kf[t] = bf16x8{};
      vf[t] = bf16x8{};
    }
  }
  wait_all();

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dk[i] = dv[i] = f32x16{};
  const float c = p.scale * kLog2e;
  int tlo[DB], thi[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tlo[db] = tr_off<D>(lane, db, 0);
    thi[db] = tr_off<D>(lane, db, 1);
  }
  const int lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * G::LOADS * 1024);
  const int lds_rw = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::RW0);
  // Tile loads: instruction n of wave w fills chunks P = (w LOADS + n) 64 + lane,
  // row r = P / KCH (RPI rows per instruction).  The swizzle repeats every PER
  // instructions, so the lane part is one of PER (row, chunk) pairs and the
  // rest is a scalar row offset.
  constexpr int RPI = 64 / G::KCH;
  constexpr int PER = 16 / RPI;

  // The (query head, query tile) pairs of this key tile, flattened; pair
  // n + 1 is staged into the other buffer while pair n is computed.
  auto col_of = [&](int hi) INLINE -> int {
    return (mb * p.mh + (p.mh == 1 ? 0 : g * p.group + hi)) * p.nkt + kt;
  };
  // (list, count and block-state entries by scalar loads, as in k_bwd_dkdv8)
  auto count_of = [&](int hi) INLINE -> int { return sload_wait(p.col_count + col_of(hi)); };
  auto entry_of = [&](int hi, int i) INLINE -> int {
    return sload_wait(p.col_list + (int64_t)col_of(hi) * p.nqt + i);
  };
  // Bitmap: this wave's 64 x 64 block of the staged pair and, when PARTIAL,
  // its 64 row words loaded into the stage's slot of this wave.
  int st_next = FMASK_SKIP;
  const int lds_bw = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::BW0 + w * 512);
  auto stage = [&](int hi, int i, int buf) INLINE {
    const int h = g * p.group + hi;
    const int qt = entry_of(hi, i) & 0x7fffffff;
    const __bf16* Q = (const __bf16*)p.q + b * p.qs[0] + h * p.qs[1];
    const __bf16* dO = (const __bf16*)p.dout + b * p.os[0] + h * p.os[1];
    const float* ws = p.ws + ((int64_t)b * p.hq + h) * p.sq * 2;
    const rsrc_t qrs = make_rsrc(Q, ((int64_t)(p.sq - 1) * p.qs[2] + D) * 2);
    const rsrc_t ors = make_rsrc(dO, ((int64_t)(p.sq - 1) * p.os[2] + D) * 2);
    const rsrc_t wrs = make_rsrc(ws, (int64_t)p.sq * 8);
    const int base = lds_w + buf * G::STAGE;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) {
      // scalar part: rows of whole swizzle periods (a multiple of 16) + tile base;
      // lane part: row tr (< 16) and its swizzled chunk
      const int rs = qt * BM + (w * G::LOADS + n - n % PER) * RPI;
      const int tr = (n % PER) * RPI + lane / G::KCH;
      const int tc = ((lane % G::KCH) ^ sw<G::KCH>(tr)) * 16;
      dma16s(qrs, (int)(tr * p.qs[2] * 2) + tc, (int)(rs * p.qs[2] * 2), base + G::Q0 + n * 1024);
      dma16s(ors, (int)(tr * p.os[2] * 2) + tc, (int)(rs * p.os[2] * 2), base + G::DO0 + n * 1024);
    }
    // 128 rows x 8 bytes = 1 KB of row values, one 16-byte load per lane of wave 0
    if (w == 0) dma16(wrs, (qt * BM * 2 + lane * 4) * 4, lds_rw + buf * G::STAGE);
    if constexpr (KIND == FMASK_ENC_BITMAP) {
      const int bi = 2 * qt + rw;
      int st = FMASK_SKIP;
      if (bi < p.nbq) {
        const int64_t x = ((int64_t)(mb * p.mh + (p.mh == 1 ? 0 : h)) * p.nbq + bi) * p.nbk + kt;
        st = sload_byte(p.bstate + x);
        if (st == FMASK_PARTIAL) {
          const int pool = sload_wait(p.bindex + x);
          if (lane < 32) dma16(make_rsrc(p.bbits + (int64_t)pool * 64, 512), lane * 16, lds_bw + buf * 4 * 512);
        }
      }
      st_next = st;
    }
  };

  int hi = 0;
  while (hi < p.group && count_of(hi) == 0) ++hi;
  int us = 0, ue = 0x7fffffff, ls = 0, le = 0;  // this lane's key column (past skv: all masked)
  int iv_head = -1;
  if (hi < p.group) {
    int i = 0, buf = 0;
    stage(hi, i, 0);
    int st_cur = st_next;
    wait_all();
    barrier();
    while (true) {
      int nh = hi, ni = i + 1;
      while (nh < p.group && ni >= count_of(nh)) { ++nh; ni = 0; }
      const bool more = nh < p.group;
      // intervals of this lane's key for the current head's mask (loaded
      // before the next stage's loads are in flight)
      const int mhh = p.mh == 1 ? 0 : g * p.group + hi;
      if (KIND != FMASK_ENC_BITMAP && mhh != iv_head) {
        iv_head = mhh;
        if (key < p.skv) {
          const int32_t* ivcol = p.iv + ((size_t)mb * p.mh + mhh) * 4 * (size_t)p.skv;
          us = ivcol[key];
          ue = ivcol[p.skv + key];
          ls = ivcol[2 * (size_t)p.skv + key];
          le = ivcol[3 * (size_t)p.skv + key];
        }
        wait_all();
      }
      const int e = entry_of(hi, i);
      if (more) stage(nh, ni, buf ^ 1);
      const int qt = e & 0x7fffffff;

      const char* qb = smem + buf * G::STAGE + G::Q0;
      const char* ob = smem + buf * G::STAGE + G::DO0;
      const float* rv = (const float*)(smem + buf * G::STAGE + G::RW0);
      // this wave: keys key (lane), rows qt*BM + rw*64 + [0, 64)
      const int ra = qt * BM + rw * 64;
      const int na = min(max(p.sq - ra, 0), 64);
      // PARTIAL: bit r of `keep` says row ra + r (r < 64, after the shift by
      // 4 half the bit of the row 4 half + r) is visible to this lane's key;
      // built once per query tile
      bool wskip, full;
      uint64_t keep = 0;
      if constexpr (KIND == FMASK_ENC_BITMAP) {
        // the wave's 64 rows are one block row: its 64 x 64 block of this key tile
        const int st = st_cur;
        wskip = st == FMASK_SKIP;
        full = st == FMASK_FULL && (kt + 1) * BN <= p.skv && na == 64;
        if (!wskip && !full) {
          uint64_t colw = 0;  // the rows that see this lane's key
          if (st == FMASK_PARTIAL) {
            // lane r holds the block's row word r; one ballot per key of this
            // wave's half gathers that key's column
            const uint64_t roww = *(const uint64_t*)(smem + G::BW0 + (buf * 4 + w) * 512 + lane * 8);
#pragma unroll 4
            for (int kk = 0; kk < 32; ++kk) {
              const uint64_t cw = __ballot((roww >> (kw * 32 + kk)) & 1ull);
              colw = l32 == kk ? cw : colw;
            }
          } else {  // FULL block with rows past sq or keys past skv
            colw = key < p.skv ? (na >= 64 ? ~0ull : ((1ull << na) - 1ull)) : 0ull;
          }
          keep = colw >> (4 * half);
        }
      } else {
        // from the key's two runs and the end of Q
        const int cm = overlap(ra, ra + na, us, ue) + overlap(ra, ra + na, ls, le);
        wskip = __ballot(!(key < p.skv) || cm == na) == ~0ull;
        full = (e & (int)FMASK_LIST_FULL_BIT) && (kt + 1) * BN <= p.skv && na == 64;
        if (!wskip && !full) {
          auto rows = [&](int a, int b) -> uint64_t {  // bits [a - ra, b - ra) within [0, 64)
            const int lo = min(max(a - ra, 0), 64), hi = min(max(b - ra, 0), 64);
            const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
            const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
            return below_hi & ~below_lo;
          };
          keep = ~(rows(us, ue) | rows(ls, le) | rows(p.sq, ra + 64)) >> (4 * half);
        }
      }
      // 0 where row offset `pos` of this lane (pos = 32 rb + 8 (r / 4) + r % 4)
      // is masked, all ones where it is visible
      auto keep_bits = [&](int pos) INLINE -> int32_t {
        const uint32_t wd = pos < 32 ? (uint32_t)keep : (uint32_t)(keep >> 32);
        return __builtin_amdgcn_sbfe((int32_t)wd, pos & 31, 1);
      };
      if (!wskip) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int lr0 = rw * 64 + rb * 32;  // first tile row of this block
          // S = Q K^T, then dP = dO V^T: 2 KT MFMAs, each A fragment read
          // kAhead MFMAs ahead into a ring of registers (one wave per SIMD:
          // nothing else hides the LDS latency)
          f32x16 s = f32x16{}, dp = f32x16{};
          {
            auto frag = [&](int n) INLINE -> bf16x8 {
              const char* tb = n < KT ? qb : ob;
              return *(const bf16x8*)(tb + chunk_off<D>(lr0 + l32, 2 * (n % KT) + half));
            };
            bf16x8 fr[kAhead];
#pragma unroll
            for (int n = 0; n < kAhead; ++n) fr[n] = frag(n);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < 2 * KT; ++n) {
              const bf16x8 a = fr[n % kAhead];
              if (n < KT) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[n], s, 0, 0, 0);
              else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[n - KT], dp, 0, 0, 0);
              if (n + kAhead < 2 * KT) fr[n % kAhead] = frag(n + kAhead);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // P, dS: lane = key, rows lr0 + 8 (r / 4) + 4 half + r % 4
          bf16x8 pb[2], sb[2];
#pragma unroll
          for (int tp = 0; tp < 2; ++tp) {
            f32x8 xp, xs;
#pragma unroll
            for (int j4 = 0; j4 < 2; ++j4) {
              const int rl = lr0 + 8 * (2 * tp + j4) + 4 * half;  // 4 consecutive rows
              const f32x4 d4 = *(const f32x4*)(rv + 2 * rl);       // {D, LSE2} x 2
              const f32x4 d5 = *(const f32x4*)(rv + 2 * rl + 4);
              const float dl[4] = {d4[0], d4[2], d5[0], d5[2]};
              const float ll[4] = {d4[1], d4[3], d5[1], d5[3]};
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                const int r = 8 * tp + 4 * j4 + q4;
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -ll[q4]));
                xp[4 * j4 + q4] = pr;
                xs[4 * j4 + q4] = pr * (dp[r] - dl[q4]);
              }
            }
            // element masks of a PARTIAL tile, in one pass over the 8 values
            // (one uniform branch rather than one per element): a masked
            // value's bits are cleared, i.e. it becomes +0
            if (!full) {
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int32_t k = keep_bits(32 * rb + 8 * (2 * tp + j / 4) + j % 4);
                xp[j] = __int_as_float(__float_as_int(xp[j]) & k);
                xs[j] = __int_as_float(__float_as_int(xs[j]) & k);
              }
            }
            pb[tp] = __builtin_convertvector(xp, bf16x8);
            sb[tp] = __builtin_convertvector(xs, bf16x8);
          }
          // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the 32 rows)
          // (MFMA m: db = m / 4, ks = m / 2 % 2, dV for even m and dK for odd
          // m; its transposed fragment read kAhead MFMAs ahead)
          {
            auto frag = [&](int m) INLINE -> bf16x8 {
              const int db = m / 4, ks = (m / 2) % 2;
              return tr_frag<D>((m & 1) ? qb : ob, lr0 + 16 * ks, tlo[db], thi[db]);
            };
            bf16x8 fr[kAhead];
#pragma unroll
            for (int m = 0; m < kAhead; ++m) fr[m] = frag(m);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < 4 * DB; ++m) {
              const int db = m / 4, ks = (m / 2) % 2;
              const bf16x8 a = fr[m % kAhead];
              if (m & 1) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[ks], dk[db], 0, 0, 0);
              else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], dv[db], 0, 0, 0);
              if (m + kAhead < 4 * DB) fr[m % kAhead] = frag(m + kAhead);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      }
      wait_all();  // the next pair landed; every wave is done with this one
      barrier();
      if (!more) break;
      hi = nh;
      i = ni;
      buf ^= 1;
      st_cur = st_next;
    }
  }

  // Sum the two row halves (waves kw and kw + 2) through LDS, then write.
  float* red = (float*)smem;  // [2 kw][2 tensors][DB][16][64] floats
  auto slot = [&](int t, int db, int r) INLINE -> float& {
    return red[(((kw * 2 + t) * DB + db) * 16 + r) * 64 + lane];
  };
  __syncthreads();
  if (rw == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        slot(0, db, r) = dk[db][r];
        slot(1, db, r) = dv[db][r];
      }
  }
  __syncthreads();
  if (rw == 0 && key < p.skv) {
    __bf16* dK = (__bf16*)p.dk + b * p.ks[0] + g * p.ks[1] + key * p.ks[2];
    __bf16* dV = (__bf16*)p.dv + b * p.vs[0] + g * p.vs[1] + key * p.vs[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 xk, xv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * rg + j;
          xk[j] = (dk[db][r] + slot(0, db, r)) * p.scale;
          xv[j] = dv[db][r] + slot(1, db, r);
        }
        const int d0 = db * 32 + 8 * rg + 4 * half;
        *(bf16x4*)(dK + d0) = __builtin_convertvector(xk, bf16x4);
        *(bf16x4*)(dV + d0) = __builtin_convertvector(xv, bf16x4);
      }
    }
  }
#endif
}

// Eight-wave form: 2 key halves x 4 row quarters of each query tile, two waves
// per SIMD.  K stays in registers as the B operand of S = Q K^T; V is staged
// once into LDS and read as the B operand of dP = dO V^T, which leaves each
// wave within 256 registers (the four-wave form keeps V in registers too and
// needs more than 256).  The four row quarters' dK and dV are summed through
// LDS at the end, in two rounds.
template <int D>
struct GeoKV8 {
  static constexpr int KCH = D / 8;
  static constexpr int TILE = BM * D * 2;        // one [128 rows][D] bf16 tile
  static constexpr int Q0 = 0, DO0 = TILE;       // Q tile, dO tile
  static constexpr int RW0 = 2 * TILE;           // [128 rows] x {D_i, LSE2_i}
  static constexpr int STAGE = RW0 + BM * 8;     // two stages (double-buffered)
  static constexpr int V0 = 2 * STAGE;           // V tile [64 keys][D]
  static constexpr int BW0 = V0 + BN * D * 2;    // bitmap: [2 stages][8 waves] x 64 row words
  static constexpr int END = BW0 + 2 * 8 * 512;
  static constexpr int LOADS = BM * KCH / 512;   // 16-byte loads per wave and tile
  static constexpr int RED = 2 * 2 * 2 * (D / 32) * 16 * 64 * 4;  // 2 quarters x 2 key halves x dK, dV
};
static_assert(GeoKV8<128>::END <= 160 * 1024 && GeoKV8<128>::RED <= GeoKV8<128>::END, "LDS");
static_assert(GeoKV8<64>::RED <= GeoKV8<64>::END, "LDS");

template <int D, int KIND>
__global__ void __launch_bounds__(512, 1) k_bwd_dkdv8(BwdParams p, int expand, int n_items) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using G = GeoKV8<D>;
  constexpr int DB = D / 32, KT = D / 16;
  constexpr int kA = 2, kV = 1;  // read-ahead of the A fragments and of the V fragments
  __shared__ __attribute__((aligned(1024))) char smem[G::END];

  const int l = blockIdx.x;
  if (l >= n_items) return;
  int col, b, g;
  kv_item(p, expand, l, &col, &b, &g);
  // (uniform, so that list and block-state reads below are scalar loads)
  col = __builtin_amdgcn_readfirstlane(col);
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  const int kt = col % p.nkt;
  const int mb = (p.mb == 1) ? 0 : b;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = w & 1, rw = w >> 1;  // key half (32 keys), 32-row quarter of each query tile
  const int half = lane >> 5, l32 = lane & 31;
  const int key = kt * BN + kw * 32 + l32;  // this lane's key (as MFMA column)

  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + g * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + g * p.vs[1];

  // V tile into LDS under the row swizzle (zeros past skv)
  char* vt = smem + G::V0;
  for (int idx = tid; idx < BN * G::KCH; idx += 512) {
    const int r = idx / G::KCH, ch = idx % G::KCH, kk = kt * BN + r;
    i32x4 x = i32x4{0, 0, 0, 0};
    if (kk < p.skv) x = *(const i32x4*)(V + kk * p.vs[2] + ch * 8);
    *(i32x4*)(vt + chunk_off<D>(r, ch)) = x;
  }
  // K as the B operand of S = Q K^T (lane: key, 8 d)
  bf16x8 kf[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
    kf[t] = key < p.skv ? *(const bf16x8*)(K + key * p.ks[2] + 16 * t + 8 * half) : bf16x8{};
  wait_all();

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dk[i] = dv[i] = f32x16{};
  const float c = p.scale * kLog2e;
  // transposing-read offsets of d-block 0; d-block db's are these XOR
  // db << 6 (the swizzle only XORs chunk bits, and db is chunk bits 2 - 3)
  const int tlo0 = tr_off<D>(lane, 0, 0), thi0 = tr_off<D>(lane, 0, 1);
  const int lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * G::LOADS * 1024);
  const int lds_rw = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::RW0);
  constexpr int RPI = 64 / G::KCH;
  constexpr int PER = 16 / RPI;

  auto col_of = [&](int hi) INLINE -> int {
    return (mb * p.mh + (p.mh == 1 ? 0 : g * p.group + hi)) * p.nkt + kt;
  };
  // List and count entries are read with scalar loads: they wait on the
  // scalar counter only, never on the vector-memory counter that the tile
  // loads in flight hold up.
  auto count_of = [&](int hi) INLINE -> int { return sload_wait(p.col_count + col_of(hi)); };
  auto entry_of = [&](int hi, int i) INLINE -> int {
    return sload_wait(p.col_list + (int64_t)col_of(hi) * p.nqt + i);
  };
  // Bitmap: this wave's 64 x 64 block of the staged pair (state read with a
  // scalar load) and, when PARTIAL, its 64 row words loaded into the stage's
  // slot of this wave.
  int st_next = FMASK_SKIP;
  const int lds_bw = __builtin_amdgcn_readfirstlane(lds_addr(smem) + G::BW0 + w * 512);
  auto stage = [&](int hi, int i, int buf) INLINE {
    const int h = g * p.group + hi;
    const int qt = entry_of(hi, i) & 0x7fffffff;
    const __bf16* Q = (const __bf16*)p.q + b * p.qs[0] + h * p.qs[1];
    const __bf16* dO = (const __bf16*)p.dout + b * p.os[0] + h * p.os[1];
    const float* ws = p.ws + ((int64_t)b * p.hq + h) * p.sq * 2;
    const rsrc_t qrs = make_rsrc(Q, ((int64_t)(p.sq - 1) * p.qs[2] + D) * 2);
    const rsrc_t ors = make_rsrc(dO, ((int64_t)(p.sq - 1) * p.os[2] + D) * 2);
    const rsrc_t wrs = make_rsrc(ws, (int64_t)p.sq * 8);
    const int base = lds_w + buf * G::STAGE;
#pragma unroll
    for (int n = 0; n < G::LOADS; ++n) {
      const int rs = qt * BM + (w * G::LOADS + n - n % PER) * RPI;
      const int tr = (n % PER) * RPI + lane / G::KCH;
      const int tc = ((lane % G::KCH) ^ sw<G::KCH>(tr)) * 16;
      dma16s(qrs, (int)(tr * p.qs[2] * 2) + tc, (int)(rs * p.qs[2] * 2), base + G::Q0 + n * 1024);
      dma16s(ors, (int)(tr * p.os[2] * 2) + tc, (int)(rs * p.os[2] * 2), base + G::DO0 + n * 1024);
    }
    if (w == 0) dma16(wrs, (qt * BM * 2 + lane * 4) * 4, lds_rw + buf * G::STAGE);
    if constexpr (KIND == FMASK_ENC_BITMAP) {
      const int slice = mb * p.mh + (p.mh == 1 ? 0 : h);
      const int bi = 2 * qt + (rw >> 1);
      int st = FMASK_SKIP;
      if (bi < p.nbq) {
        const int64_t x = ((int64_t)slice * p.nbq + bi) * p.nbk + kt;
        st = sload_byte(p.bstate + x);
        if (st == FMASK_PARTIAL) {
          const int pool = sload_wait(p.bindex + x);
          const rsrc_t brs = make_rsrc(p.bbits + (int64_t)pool * 64, 512);
          if (lane < 32) dma16(brs, lane * 16, lds_bw + buf * 8 * 512);
        }
      }
      st_next = st;
    }
  };

  int hi = 0;
  while (hi < p.group && count_of(hi) == 0) ++hi;
  int us = 0, ue = 0x7fffffff, ls = 0, le = 0;  // this lane's key column (past skv: all masked)
  int iv_head = -1;
  if (hi < p.group) {
    int i = 0, buf = 0;
    stage(hi, i, 0);
    int st_cur = st_next;
    wait_all();
    barrier();
    while (true) {
      int nh = hi, ni = i + 1;
      while (nh < p.group && ni >= count_of(nh)) { ++nh; ni = 0; }
      const bool more = nh < p.group;
      const int mhh = p.mh == 1 ? 0 : g * p.group + hi;
      if (KIND != FMASK_ENC_BITMAP && mhh != iv_head) {
        iv_head = mhh;
        if (key < p.skv) {
          const int32_t* ivcol = p.iv + ((size_t)mb * p.mh + mhh) * 4 * (size_t)p.skv;
          us = ivcol[key];
          ue = ivcol[p.skv + key];
          ls = ivcol[2 * (size_t)p.skv + key];
          le = ivcol[3 * (size_t)p.skv + key];
        }
        wait_all();
      }
      const int e = entry_of(hi, i);
      if (more) stage(nh, ni, buf ^ 1);
      const int qt = e & 0x7fffffff;

      const char* qb = smem + buf * G::STAGE + G::Q0;
      const char* ob = smem + buf * G::STAGE + G::DO0;
      const float* rv = (const float*)(smem + buf * G::STAGE + G::RW0);
      // this wave: keys key (lane), rows ra + [0, 32)
      const int ra = qt * BM + rw * 32;
      const int na = min(max(p.sq - ra, 0), 32);
      // PARTIAL: bit 8 (j / 4) + j % 4 of `keep` says whether value j of this
      // lane (row ra + 8 (j / 4) + 4 half + j % 4) is visible to its key
      bool wskip, full;
      uint32_t keep = 0;
      if constexpr (KIND == FMASK_ENC_BITMAP) {
        // the wave's 32 rows are one half of a 64-row block row
        const int st = st_cur;
        wskip = st == FMASK_SKIP || na == 0;
        full = st == FMASK_FULL && (kt + 1) * BN <= p.skv && na == 32;
        if (!wskip && !full) {
          uint64_t colw = 0;  // the block's rows that see this lane's key
          if (st == FMASK_PARTIAL) {
            const uint64_t roww = *(const uint64_t*)(smem + G::BW0 + (buf * 8 + w) * 512 + lane * 8);
#pragma unroll 4
            for (int kk = 0; kk < 32; ++kk) {
              const uint64_t cw = __ballot((roww >> (kw * 32 + kk)) & 1ull);
              colw = l32 == kk ? cw : colw;
            }
          } else {  // FULL block with rows past sq or keys past skv
            colw = key < p.skv ? ((na >= 32 ? 0xffffffffull : ((1ull << na) - 1ull)) << (32 * (rw & 1))) : 0ull;
          }
          keep = (uint32_t)(colw >> (32 * (rw & 1))) >> (4 * half);
        }
      } else {
        const int cm = overlap(ra, ra + na, us, ue) + overlap(ra, ra + na, ls, le);
        wskip = __ballot(!(key < p.skv) || cm == na) == ~0ull;
        full = (e & (int)FMASK_LIST_FULL_BIT) && (kt + 1) * BN <= p.skv && na == 32;
        if (!wskip && !full) {
          auto rows = [&](int a, int b) -> uint32_t {  // bits [a - ra, b - ra) within [0, 32)
            const int lo = min(max(a - ra, 0), 32), hi = min(max(b - ra, 0), 32);
            const uint32_t below_hi = hi >= 32 ? ~0u : ((1u << hi) - 1u);
            const uint32_t below_lo = lo >= 32 ? ~0u : ((1u << lo) - 1u);
            return below_hi & ~below_lo;
          };
          keep = ~(rows(us, ue) | rows(ls, le) | rows(p.sq, ra + 32)) >> (4 * half);
        }
      }
      if (!wskip) {
        const int lr0 = rw * 32;  // first tile row of this wave
        // S = Q K^T, then dP = dO V^T: A fragments read kA MFMAs ahead, V
        // fragments kV ahead
        f32x16 s = f32x16{}, dp = f32x16{};
        {
          auto afrag = [&](int n) INLINE -> bf16x8 {
            const char* tb = n < KT ? qb : ob;
            return *(const bf16x8*)(tb + chunk_off<D>(lr0 + l32, 2 * (n % KT) + half));
          };
          auto vfrag = [&](int j) INLINE -> bf16x8 {
            return *(const bf16x8*)(vt + chunk_off<D>(kw * 32 + l32, 2 * j + half));
          };
          bf16x8 fr[kA], vr[kV];
#pragma unroll
          for (int n = 0; n < kA; ++n) fr[n] = afrag(n);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int n = 0; n < 2 * KT; ++n) {
            const bf16x8 a = fr[n % kA];
            if (n < KT) {
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[n], s, 0, 0, 0);
            } else {
              const int j = n - KT;
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vr[j % kV], dp, 0, 0, 0);
              if (j + kV < KT) vr[j % kV] = vfrag(j + kV);
            }
            if (n + kA < 2 * KT) fr[n % kA] = afrag(n + kA);
            if (n + kV == KT) {
#pragma unroll
              for (int j = 0; j < kV; ++j) vr[j] = vfrag(j);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // P, dS: lane = key, rows lr0 + 8 (r / 4) + 4 half + r % 4
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          f32x8 xp, xs;
#pragma unroll
          for (int j4 = 0; j4 < 2; ++j4) {
            const int rl = lr0 + 8 * (2 * tp + j4) + 4 * half;  // 4 consecutive rows
            const f32x4 d4 = *(const f32x4*)(rv + 2 * rl);       // {D, LSE2} x 2
            const f32x4 d5 = *(const f32x4*)(rv + 2 * rl + 4);
            const float dl[4] = {d4[0], d4[2], d5[0], d5[2]};
            const float ll[4] = {d4[1], d4[3], d5[1], d5[3]};
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int r = 8 * tp + 4 * j4 + q4;
              const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -ll[q4]));
              xp[4 * j4 + q4] = pr;
              xs[4 * j4 + q4] = pr * (dp[r] - dl[q4]);
            }
          }
          // element masks of a PARTIAL tile in one pass over the 8 values: a
          // masked value's bits are cleared (it becomes +0)
          if (!full) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int32_t k = __builtin_amdgcn_sbfe((int32_t)keep, 8 * (2 * tp + j / 4) + j % 4, 1);
              xp[j] = __int_as_float(__float_as_int(xp[j]) & k);
              xs[j] = __int_as_float(__float_as_int(xs[j]) & k);
            }
          }
          pb[tp] = __builtin_convertvector(xp, bf16x8);
          sb[tp] = __builtin_convertvector(xs, bf16x8);
        }
        // dV^T += dO^T P,  dK^T += Q^T dS  (contraction over the 32 rows;
        // MFMA m: db = m / 4, ks = m / 2 % 2, dV for even m and dK for odd m)
        {
          auto frag = [&](int m) INLINE -> bf16x8 {
            const int db = m / 4, ks = (m / 2) % 2;
            return tr_frag<D>((m & 1) ? qb : ob, lr0 + 16 * ks, tlo0 ^ (db << 6), thi0 ^ (db << 6));
          };
          bf16x8 fr[kAhead];
#pragma unroll
          for (int m = 0; m < kAhead; ++m) fr[m] = frag(m);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int m = 0; m < 4 * DB; ++m) {
            const int db = m / 4, ks = (m / 2) % 2;
            const bf16x8 a = fr[m % kAhead];
            if (m & 1) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[ks], dk[db], 0, 0, 0);
            else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], dv[db], 0, 0, 0);
            if (m + kAhead < 4 * DB) fr[m % kAhead] = frag(m + kAhead);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wait_all();  // the next pair landed; every wave is done with this one
      barrier();
      if (!more) break;
      hi = nh;
      i = ni;
      buf ^= 1;
      st_cur = st_next;
    }
  }

  // Sum the four row quarters (waves kw, kw + 2, kw + 4, kw + 6) through LDS
  // in two rounds, then write.
  float* red = (float*)smem;  // [2 quarters][2 kw][2 tensors][DB][16][64] floats
  auto slot = [&](int q, int t, int db, int r) INLINE -> float& {
    return red[((((q * 2 + kw) * 2 + t) * DB + db) * 16 + r) * 64 + lane];
  };
  __syncthreads();
  if (rw >= 2) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        slot(rw - 2, 0, db, r) = dk[db][r];
        slot(rw - 2, 1, db, r) = dv[db][r];
      }
  }
  __syncthreads();
  if (rw < 2) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[db][r] += slot(rw, 0, db, r);
        dv[db][r] += slot(rw, 1, db, r);
      }
  }
  __syncthreads();
  if (rw == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        slot(0, 0, db, r) = dk[db][r];
        slot(0, 1, db, r) = dv[db][r];
      }
  }
  __syncthreads();
  if (rw == 0 && key < p.skv) {
    __bf16* dK = (__bf16*)p.dk + b * p.ks[0] + g * p.ks[1] + key * p.ks[2];
    __bf16* dV = (__bf16*)p.dv + b * p.vs[0] + g * p.vs[1] + key * p.vs[2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 xk, xv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * rg + j;
          xk[j] = (dk[db][r] + slot(0, 0, db, r)) * p.scale;
          xv[j] = dv[db][r] + slot(0, 1, db, r);
        }
        const int d0 = db * 32 + 8 * rg + 4 * half;
        *(bf16x4*)(dK + d0) = __builtin_convertvector(xk, bf16x4);
        *(bf16x4*)(dV + d0) = __builtin_convertvector(xv, bf16x4);
      }
    }
  }
#endif
}

template <int D, int KIND>
hipError_t launch_d(const BwdParams& p, hipStream_t s) {
  // (With no query row the dK / dV kernel still runs: its empty column lists
  // write zeros.  With no key the dQ kernel's empty lists do the same.)
  hipError_t e = hipSuccess;
  // dQ (and the rows' D_i, LSE_i for the dK / dV kernel): items like the
  // forward (tile rows x (batch, head) expansion)
  {
    const int expand = (p.mb == 1 ? p.b : 1) * (p.mh == 1 ? p.hq : 1);
    const int64_t n = (int64_t)p.mb * p.mh * p.nqt * expand;
    const int gsz = (p.mh == 1) ? p.group : 1;
    const int64_t unit = (int64_t)kXcds * gsz;
    const int64_t npad = (n + unit - 1) / unit * unit;
    if (n > 0)
      hipLaunchKernelGGL((k_bwd_dq<D, KIND>), dim3((unsigned)npad), dim3(256), 0, s, p, expand, (int)n, gsz);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dK, dV: one item per (key tile column, batch, K/V head)
  {
    int expand;
    int64_t n;
    if (p.mh == 1) {
      expand = (p.mb == 1 ? p.b : 1) * p.hkv;
      n = (int64_t)p.mb * p.nkt * expand;
    } else {
      expand = 1;
      n = (int64_t)p.b * p.hkv * p.nkt;
    }
    // D = 128: eight waves (two per SIMD, V in LDS); D = 64: four waves, whose
    // 66 KB of LDS already let two workgroups share a CU
    if (n > 0) {
      if constexpr (D == 128)
        hipLaunchKernelGGL((k_bwd_dkdv8<D, KIND>), dim3((unsigned)n), dim3(512), 0, s, p, expand, (int)n);
      else
        hipLaunchKernelGGL((k_bwd_dkdv<D, KIND>), dim3((unsigned)n), dim3(256), 0, s, p, expand, (int)n);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdParams& p, int32_t d, hipStream_t s) {
  if (p.bm != BM || p.bn != BN) return hipErrorInvalidValue;
  if (p.kind == FMASK_ENC_BITMAP) {
    if (d == 128) return launch_d<128, FMASK_ENC_BITMAP>(p, s);
    if (d == 64) return launch_d<64, FMASK_ENC_BITMAP>(p, s);
    return hipErrorInvalidValue;
  }
  if (d == 128) return launch_d<128, FMASK_ENC_INTERVALS>(p, s);
  if (d == 64) return launch_d<64, FMASK_ENC_INTERVALS>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
