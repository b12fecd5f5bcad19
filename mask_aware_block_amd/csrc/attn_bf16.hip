// Masked attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Work unit: one bm x d query tile of one (batch, q head), bm = 32 * NW rows
// (NW waves, 32 query rows per wave), walking the compact list of its non-SKIP
// 64-key tiles (the tile classifier's output).  FULL tiles run without any
// per-element mask; PARTIAL tiles (and the ragged last key tile) mask element
// by element from the interval or bitmap encoding.  SKIP tiles are never
// loaded.  This is the behaviour the FlashMask rebuttal page and the Binary
// Block Masking abstract ask of a mask-aware kernel; the register and LDS
// layout below is our own, designed for CDNA4.
//
// Per wave and key tile:
//   S^T[64 keys x 32 rows] = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from
//                                     LDS, B = Q^T kept in registers.  Lane l
//                                     then holds query row (l & 31) and 32 keys,
//                                     so row max / sum stay in-lane plus one
//                                     exchange with lane l ^ 32.
//   online softmax in the exp2 domain (scale * log2(e) folded into one FMA),
//   running max starting at -FLT_MAX so exp(-inf - -inf) never happens.
//   O^T[d x 32 rows] += V^T P^T       A = V^T from LDS, B = P^T straight from
//                                     the S^T accumulators converted to bf16.
// V is written to LDS transposed (d-major) with the keys of every 16-key group
// permuted (bits 2 and 3 of the key index swapped) so that the 8 keys one lane
// needs for a PV step are contiguous: one ds_read_b128 per MFMA operand.
// K/V tiles are double-buffered in LDS; the next tile's global loads are in
// flight while the current tile is computed.  Both LDS arrays are XOR-
// swizzled in 16-byte chunks so the MFMA operand reads are conflict-free.
//
// GQA: query head h reads K/V head h / group; the group's heads of one query
// tile are consecutive work items placed on the same XCD (L2 reuse of K/V).
#include <float.h>

#include "internal.h"

namespace fmask {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int NW>
struct Cfg {
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = D * BN * 2;
  static constexpr int IV_BYTES = BN * 16;
  static constexpr int STAGE = K_BYTES + V_BYTES + IV_BYTES;
  static constexpr int KLOADS = (BN * KCH + NT - 1) / NT;        // 16-byte K chunks per thread
  static constexpr int VGROUPS = ((BN / 4) * KCH + NT - 1) / NT;  // (4 keys x 16 bytes) per thread
};

__device__ inline int swap23(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }
__device__ inline int vswz(int d) { return (d ^ (d >> 3)) & 7; }

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

template <int D, int NW, int KIND>
__global__ void __launch_bounds__(64 * NW, 2) k_attn_tile_bf16(TileAttnParams p, int gsz) {
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int l = logical_item(gsz);
  if (l >= p.n_items) return;
  const Item it = decode_item(p, l);
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int q0 = it.qt * C::BM;
  const int qrow = q0 + w * 32 + l32;

  const __bf16* Q = (const __bf16*)p.q + it.b * p.qs[0] + it.h * p.qs[1];
  const __bf16* K = (const __bf16*)p.k + it.b * p.ks[0] + it.kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + it.b * p.vs[0] + it.kvh * p.vs[1];
  const int32_t* list = p.list + (int64_t)it.row * p.nkt;
  const int cnt = p.count[it.row];
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];

  // Q^T as MFMA B operand: lane holds row qrow, d = 16 t + 8 half + 0..7.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qrow < p.sq) qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
    else qf[t] = bf16x8{};
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = p.scale * kLog2e;

  // Bitmap encoding: this wave's 32 rows lie in one 64-row block row.
  const int brow = (q0 + w * 32) / kBlk;
  const size_t bbase = ((size_t)it.mb * p.mh + it.mh) * p.nbq;

  u32x4 kreg[C::KLOADS];
  u32x4 vreg[C::VGROUPS][4];
  i32x4 ivreg = i32x4{0, 0, 0, 0};

  // K/V of this (batch, K/V head) through buffer resources: 32-bit offsets and
  // hardware range checking (rows at or past skv read as zero).
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)K, (short)0, (int)(((int64_t)(p.skv - 1) * ks2 + D) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)V, (short)0, (int)(((int64_t)(p.skv - 1) * vs2 + D) * 2), 0x00020000);
  int koff[C::KLOADS];
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    int idx = tid + C::NT * i;
    koff[i] = (int)((idx / C::KCH) * ks2 * 2 + (idx % C::KCH) * 16);
  }
  int voff[C::VGROUPS];
#pragma unroll
  for (int i = 0; i < C::VGROUPS; ++i) {
    int g = tid + C::NT * i;
    voff[i] = (int)((4 * (g % (BN / 4))) * vs2 * 2 + (g / (BN / 4)) * 16);
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2), vrow = (int)(vs2 * 2);

  auto load_tile = [&](int kt) {
    const int key0 = kt * BN;
    const int kb0 = kt * kstep, vb0 = kt * vstep;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      if ((BN * C::KCH) % C::NT == 0 || tid + C::NT * i < BN * C::KCH)
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, koff[i] + kb0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::VGROUPS; ++i) {
      if (((BN / 4) * C::KCH) % C::NT == 0 || tid + C::NT * i < (BN / 4) * C::KCH) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i] + vb0 + j * vrow, 0, 0);
      }
    }
    if (KIND == FMASK_ENC_INTERVALS && tid < BN) {
      int key = key0 + tid;
      if (key < p.skv) {
        const int32_t* col = p.iv + ((size_t)it.mb * p.mh + it.mh) * 4 * (size_t)p.skv;
        int32_t uts = col[key], ute = col[p.skv + key];
        int32_t lts = col[2 * (size_t)p.skv + key], lte = col[3 * (size_t)p.skv + key];
        ivreg = i32x4{uts, ute - uts, lts, lte - lts};
      } else {
        ivreg = i32x4{0, 0x7fffffff, 0, 0};  // beyond the keys: masked for every row
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* kb = smem + buf * C::STAGE;
    char* vb = kb + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::KLOADS; ++i) {
      int idx = tid + C::NT * i;
      if (idx < BN * C::KCH) {
        int key = idx / C::KCH, ch = idx % C::KCH;
        *(u32x4*)(kb + key * (D * 2) + ((ch ^ (key & (C::KCH - 1))) * 16)) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::VGROUPS; ++i) {
      int g = tid + C::NT * i;
      if (g < (BN / 4) * C::KCH) {
        int kg = g % (BN / 4), ch = g / (BN / 4);
        int pos = swap23(4 * kg);
        int pch = pos >> 3, pin = (pos & 7) * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int d = ch * 8 + e;
          int m = e >> 1;
          uint32_t a0 = vreg[i][0][m], a1 = vreg[i][1][m], a2 = vreg[i][2][m], a3 = vreg[i][3][m];
          u32x2 out;
          if (e & 1) {
            out[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            out[1] = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            out[0] = (a0 & 0xffffu) | (a1 << 16);
            out[1] = (a2 & 0xffffu) | (a3 << 16);
          }
          *(u32x2*)(vb + d * (BN * 2) + ((pch ^ vswz(d)) * 16) + pin) = out;
        }
      }
    }
    if (KIND == FMASK_ENC_INTERVALS && tid < BN) *(i32x4*)(vb + C::V_BYTES + tid * 16) = ivreg;
  };

  auto compute_tile = [&](int buf, int kt, bool full) {
    const char* kb = smem + buf * C::STAGE;
    const char* vb = kb + C::K_BYTES;
    const bool ragged = (kt + 1) * BN > p.skv;

    if (q0 + w * 32 >= p.sq) return;  // every row of this wave lies past the end
    bool need_mask = !full || ragged;
    uint64_t word = ~0ull;
    if (KIND == FMASK_ENC_BITMAP) {
      uint8_t st = p.bstate[(bbase + brow) * p.nbk + kt];
      if (st == FMASK_SKIP) return;  // nothing visible in this wave's rows
      if (st == FMASK_PARTIAL) {
        int32_t idx = p.bindex[(bbase + brow) * p.nbk + kt];
        word = p.bbits[(int64_t)idx * kBlk + (qrow & (kBlk - 1))];
        need_mask = true;
      } else {
        int valid = p.skv - kt * BN;
        word = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
        need_mask = ragged;
      }
    }

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      s[kh] = f32x16{};
      const int key = kh * 32 + l32;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        int ch = 2 * t + half;
        bf16x8 a = *(const bf16x8*)(kb + key * (D * 2) + ((ch ^ (key & (C::KCH - 1))) * 16));
        s[kh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[t], s[kh], 0, 0, 0);
      }
    }

    if (need_mask) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            int key = kh * 32 + 8 * rg + 4 * half + r4;  // key index inside the tile
            bool masked;
            if (KIND == FMASK_ENC_INTERVALS) {
              i32x4 iv = *(const i32x4*)(vb + C::V_BYTES + key * 16);
              masked = ((uint32_t)(qrow - iv[0]) < (uint32_t)iv[1]) ||
                       ((uint32_t)(qrow - iv[2]) < (uint32_t)iv[3]);
            } else {
              masked = ((word >> key) & 1ull) == 0;
            }
            if (masked) s[kh][rg * 4 + r4] = -INFINITY;
          }
        }
      }
    }

    // Online softmax (row = lane's query; the other 32 keys sit in lane ^ 32).
    float mloc = s[0][0];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kh][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // Lazy rescale: the running max only moves when some row's max grows by
    // more than 8 in the exp2 domain, so p = exp2(s c - m c) stays <= 2^8.
    const float m_cand = fmaxf(m_run, mloc);
    const bool grow = (m_cand - m_run) * c > 8.f;
    if (__any(grow)) {
      const float m_new = grow ? m_cand : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }
    const float mneg = -m_run * c;
    bf16x8 pf[4];
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
    // Row sums of the bf16 probabilities actually multiplied into V.
    const bf16x2 one2 = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x2 pr = bf16x2{pf[ks][2 * j], pf[ks][2 * j + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_run, false);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = db * 32 + l32;
      const char* vrow = vb + d * (BN * 2);
      const int sw = vswz(d);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        int ch = 2 * ks + half;  // = 4 kh + 2 tp + half
        bf16x8 a = *(const bf16x8*)(vrow + ((ch ^ sw) * 16));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
      }
    }
  };

  if (cnt > 0) {
    load_tile(list[0] & 0x7fffffff);
    store_tile(0);
  }
  __syncthreads();
  for (int i = 0; i < cnt; ++i) {
    const uint32_t e = (uint32_t)list[i];
    const int kt = (int)(e & 0x7fffffffu);
    const bool full = (e & FMASK_LIST_FULL_BIT) != 0;
    const bool more = i + 1 < cnt;
    if (more) load_tile(list[i + 1] & 0x7fffffff);
    compute_tile(i & 1, kt, full);
    if (more) store_tile((i + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = O / l, zero rows for l = 0, LSE in natural log.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.sq) {
    __bf16* O = (__bf16*)p.o + it.b * p.os[0] + it.h * p.os[1] + qrow * p.os[2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        int d0 = db * 32 + 8 * rg + 4 * half;
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        f32x4 x = f32x4{acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2],
                        acc[db][4 * rg + 3]} * inv;
        *(bf16x4*)(O + d0) = __builtin_convertvector(x, bf16x4);
      }
    }
    if (p.lse && half == 0) {
      float lse = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
      p.lse[((int64_t)it.b * p.hq + it.h) * p.sq + qrow] = lse;
    }
  }
}

template <int D, int NW>
hipError_t launch_dn(const TileAttnParams& p, hipStream_t s) {
  int gsz = (p.mh == 1) ? p.group : 1;
  if (p.n_items <= 0) return hipSuccess;
  int64_t unit = (int64_t)kXcds * gsz;
  int64_t npad = (p.n_items + unit - 1) / unit * unit;
  if (p.kind == FMASK_ENC_INTERVALS)
    hipLaunchKernelGGL((k_attn_tile_bf16<D, NW, FMASK_ENC_INTERVALS>), dim3((unsigned)npad),
                       dim3(64 * NW), 0, s, p, gsz);
  else
    hipLaunchKernelGGL((k_attn_tile_bf16<D, NW, FMASK_ENC_BITMAP>), dim3((unsigned)npad),
                       dim3(64 * NW), 0, s, p, gsz);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_tile_bf16(const TileAttnParams& p, int32_t d, hipStream_t s) {
  if (p.bn != BN) return hipErrorInvalidValue;
  if (d == 128 && p.bm == 128) return launch_dn<128, 4>(p, s);
  if (d == 128 && p.bm == 64) return launch_dn<128, 2>(p, s);
  if (d == 64 && p.bm == 128) return launch_dn<64, 4>(p, s);
  if (d == 64 && p.bm == 64) return launch_dn<64, 2>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
