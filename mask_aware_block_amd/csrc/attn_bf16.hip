// Masked attention forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Work unit: one bm x d query tile of one (batch, q head), bm = 32 * NW rows
// (NW waves, 32 query rows per wave), walking the compact list of its non-SKIP
// 64-key tiles (the tile classifier's output).  FULL tiles run without any
// per-element mask; PARTIAL tiles (and the ragged last key tile) mask element
// by element from the interval or bitmap encoding.  SKIP tiles are never
// loaded.  This is the behaviour the FlashMask rebuttal page and the Binary
// Block Masking abstract ask of a mask-aware kernel; the register and LDS
// layout below is our own, designed for CDNA4 (gfx950).
//
// Per wave and key tile:
//   S^T[64 keys x 32 rows] = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from
//                                     LDS, B = Q^T kept in registers.  Lane l
//                                     then holds query row (l & 31) and 32 keys,
//                                     so row max / sum stay in-lane plus one
//                                     exchange with lane l ^ 32.
//   online softmax in the exp2 domain (scale * log2(e) folded into one FMA),
//   running max from -FLT_MAX (exp(-inf - -inf) never happens), moved only
//   when a row's max grows by more than 8 (exp2 units), so the O rescale is
//   rare; row sums are taken over the bf16 probabilities fed to the MFMA.
//   O^T[d x 32 rows] += V^T P^T       A = V^T fragments read from the row-major
//                                     V tile with the gfx950 transposing LDS
//                                     read (ds_read_b64_tr_b16), B = P^T taken
//                                     straight from the S^T accumulators.
// K and V tiles go from HBM to LDS with direct-to-LDS buffer loads (no VGPR
// staging), double-buffered: the next tile's loads are in flight while the
// current one is computed.  Buffer range checking turns rows past the end of
// the sequence into zeros.  Both LDS tiles are XOR-swizzled in 16-byte chunks
// (the swizzle is applied through the global addresses each lane loads), so
// the MFMA operand reads are free of bank conflicts.
//
// GQA: query head h reads K/V head h / group; the group's heads of one query
// tile are consecutive work items placed on the same XCD (L2 reuse of K/V).
#include <float.h>

#include "device_util.h"
#include "internal.h"

namespace fmask {
namespace {

// A wave-uniform 64-bit value in scalar registers (both halves read from the
// first active lane).
__device__ inline int64_t rfl64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS FMASK_LDS_AS

constexpr int BN = 64;
constexpr int kListLds = 2048;  // tile-list entries staged in LDS
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int NW>
struct Cfg {
  static constexpr int BM = 32 * NW;
  static constexpr int NT = 64 * NW;
  static constexpr int KCH = D / 8;                  // 16-byte chunks per row
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = BN * D * 2;
  static constexpr int IV_BYTES = BN * 16;
  static constexpr int STAGE = K_BYTES + V_BYTES + IV_BYTES;
  static constexpr int CHUNKS = BN * KCH;            // 16-byte chunks per K (or V) tile
  static constexpr int LOADS = CHUNKS / NT;          // direct-to-LDS loads per thread per tile
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the workgroup");
};

// Chunk swizzle of the K tile: conflict-free 16-byte reads of 32 rows.
template <int KCH>
__device__ inline int kswz(int key) { return key & (KCH - 1); }
// Chunk swizzle of the V tile: the transposing reads of one instruction touch
// 8 consecutive rows x 64 bytes; spread them over all banks.
template <int KCH>
__device__ inline int vswz(int key) {
  return KCH == 16 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

__device__ inline int overlap(int a0, int a1, int b0, int b1) {
  return max(0, min(a1, b1) - max(a0, b0));
}

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
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = Cfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];

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

  // Rows past the end may be read (as zeros) but never hold stale NaN bits.
  for (int i = tid; i < 2 * C::STAGE / 16; i += C::NT) ((i32x4*)smem)[i] = i32x4{0, 0, 0, 0};
  // The tile list goes to LDS once (its entries are then read without any
  // wait on the memory counters that the tile loads use).
  __shared__ int32_t lst[kListLds];
  for (int i = tid; i < min(cnt, kListLds); i += C::NT) lst[i] = list[i];
  auto entry = [&](int i) -> int {
    return i < kListLds ? __builtin_amdgcn_readfirstlane(lst[i]) : sload_wait(list + i);
  };

  // Q^T as MFMA B operand: lane holds row qrow, d = 16 t + 8 half + 0..7.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qrow < p.sq) qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
    else qf[t] = bf16x8{};
  }

  // Nothing the compiler tracks may stay pending once untracked tile loads
  // are in flight.
  wait_all();

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = p.scale * kLog2e;

  // Bitmap encoding: this wave's 32 rows lie in one 64-row block row.
  const int brow = (q0 + w * 32) / kBlk;
  const size_t bbase = ((size_t)it.mb * p.mh + it.mh) * p.nbq;

  // Buffer resources over this (batch, K/V head): 32-bit offsets, and rows at
  // or past skv fall outside the range and read as zero.
  const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);

  // Direct-to-LDS loads: instruction n of wave w fills LDS chunks
  // P = (w * LOADS + n) * 64 + lane; chunk P holds row P / KCH, physical chunk
  // P % KCH, i.e. logical chunk (P % KCH) ^ swizzle(row) of that row.
  int kgo[C::LOADS], vgo[C::LOADS];
#pragma unroll
  for (int n = 0; n < C::LOADS; ++n) {
    const int P = (w * C::LOADS + n) * 64 + lane;
    const int key = P / C::KCH, pc = P % C::KCH;
    kgo[n] = (int)(key * ks2 * 2 + ((pc ^ kswz<C::KCH>(key)) * 16));
    vgo[n] = (int)(key * vs2 * 2 + ((pc ^ vswz<C::KCH>(key)) * 16));
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2);

  // PV operand: two transposing reads per MFMA.  Lane (group g = lane / 16,
  // r = (lane % 16) / 4, c4 = lane % 4) addresses row base + 4 (g / 2) + r and
  // the 8 bytes at d = 32 db + 16 (g % 2) + 4 c4; the read hands lane l the four
  // rows at d = 32 db + (l % 32), i.e. the keys of its P^T slots.
  const int tg = lane >> 4, tr = (lane >> 2) & 3, tc4 = lane & 3;
  const int vrow_l = 4 * (tg >> 1) + tr;  // row offset of this lane inside a 16-key group
  int vofs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int ch = 4 * db + 2 * (tg & 1) + (tc4 >> 1);
    vofs[db] = vrow_l * (D * 2) + ((ch ^ vswz<C::KCH>(vrow_l)) * 16) + (tc4 & 1) * 8;
  }

  i32x4 ivreg = i32x4{0, 0, 0, 0};

  // LDS byte address where this wave's loads of stage 0 start (scalar)
  const int lds_w = __builtin_amdgcn_readfirstlane(lds_addr(smem) + w * C::LOADS * 1024);
  auto issue_tile = [&](int kt, int buf) {
    const int kb = lds_w + buf * C::STAGE, vb = kb + C::K_BYTES;
    const int kb0 = kt * kstep, vb0 = kt * vstep;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) dma16(krs, kgo[n] + kb0, kb + n * 1024);
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) dma16(vrs, vgo[n] + vb0, vb + n * 1024);
    if (KIND == FMASK_ENC_INTERVALS && tid < BN) {
      const int key = kt * BN + tid;
      if (key < p.skv) {
        const int32_t* col = p.iv + ((size_t)it.mb * p.mh + it.mh) * 4 * (size_t)p.skv;
        // raw values only: the loads stay in flight behind the tile's loads
        ivreg = i32x4{col[key], col[p.skv + key], col[2 * (size_t)p.skv + key],
                      col[3 * (size_t)p.skv + key]};
      } else {
        ivreg = i32x4{0, 0x7fffffff, 0, 0};  // past the keys: masked for every row
      }
    }
  };
  // intervals to LDS as (start, length) pairs, after the tile's compute
  auto store_iv = [&](int buf) {
    if (KIND == FMASK_ENC_INTERVALS && tid < BN)
      *(i32x4*)(smem + buf * C::STAGE + C::K_BYTES + C::V_BYTES + tid * 16) =
          i32x4{ivreg[0], ivreg[1] - ivreg[0], ivreg[2], ivreg[3] - ivreg[2]};
  };

  auto compute_tile = [&](int buf, int kt, bool full) {
    const char* kb = smem + buf * C::STAGE;
    const char* vb = kb + C::K_BYTES;
    const char* ivb = vb + C::V_BYTES;
    const bool ragged = (kt + 1) * BN > p.skv;

    bool need_mask = !full || ragged;
    uint64_t word = ~0ull;
    if (KIND == FMASK_ENC_BITMAP) {
      if (q0 + w * 32 >= p.sq) return;  // every row of this wave lies past the end
      // (state and pool entry by scalar loads: a vector load's wait would also
      // drain the next tile's loads in flight)
      const int64_t bx = rfl64((int64_t)(bbase + brow) * p.nbk + kt);
      const int st = sload_byte(p.bstate + bx);
      if (st == FMASK_SKIP) return;  // nothing visible in this wave's rows
      if (st == FMASK_PARTIAL) {
        const int32_t idx = sload_wait(p.bindex + bx);
        word = p.bbits[(int64_t)idx * kBlk + (qrow & (kBlk - 1))];
        need_mask = true;
      } else {
        int valid = p.skv - kt * BN;
        word = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
        need_mask = ragged;
      }
    }

    if (KIND == FMASK_ENC_INTERVALS && need_mask) {
      // This wave's own state for the tile (lane = key column): its 32 rows
      // may see nothing (skip the tile) or everything (no element mask).
      // Keys past skv carry an all-rows interval and count as masked.
      const i32x4 iv = *(const i32x4*)(ivb + lane * 16);
      const int a0 = q0 + w * 32, a1 = min(a0 + 32, p.sq), n = max(0, a1 - a0);
      const int cm = overlap(a0, a1, iv[0], iv[0] + iv[1]) + overlap(a0, a1, iv[2], iv[2] + iv[3]);
      if (__ballot(cm == n) == ~0ull) return;
      if (__ballot(cm != 0) == 0ull) need_mask = false;
    }

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      s[kh] = f32x16{};
      const int key = kh * 32 + l32;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const int ch = 2 * t + half;
        bf16x8 a = *(const bf16x8*)(kb + key * (D * 2) + ((ch ^ kswz<C::KCH>(key)) * 16));
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
            const int key = kh * 32 + 8 * rg + 4 * half + r4;  // key index inside the tile
            bool masked;
            if (KIND == FMASK_ENC_INTERVALS) {
              i32x4 iv = *(const i32x4*)(ivb + key * 16);
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

    // O^T += V^T P^T; P^T step ks covers keys 16 ks .. 16 ks + 15.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const char* a0 = vb + vofs[db] + (16 * ks) * (D * 2);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)a0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a0 + 8 * (D * 2)));
        bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
      }
    }
  };

  __syncthreads();  // LDS cleared and the list staged before any tile load lands
  int e_cur = 0, e_next = 0;
  if (cnt > 0) {
    e_cur = entry(0);
    if (cnt > 1) e_next = entry(1);
    issue_tile(e_cur & 0x7fffffff, 0);
    wait_all();  // tile 0 and its intervals
    store_iv(0);
  }
  wait_all();
  __syncthreads();
  for (int i = 0; i < cnt; ++i) {
    const int kt = e_cur & 0x7fffffff;
    const bool full = (e_cur & (int)FMASK_LIST_FULL_BIT) != 0;
    const bool more = i + 1 < cnt;
    int e_after = 0;
    if (more) {
      if (i + 2 < cnt) e_after = entry(i + 2);
      issue_tile(e_next & 0x7fffffff, (i + 1) & 1);
    }
    compute_tile(i & 1, kt, full);
    if (more) store_iv((i + 1) & 1);
    wait_all();  // tile i+1 landed, its intervals written
    barrier();
    e_cur = e_next;
    e_next = e_after;
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
        const int d0 = db * 32 + 8 * rg + 4 * half;
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
#endif
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
  if (d == 128 && p.bm == 256) return launch_dn<128, 8>(p, s);
  if (d == 128 && p.bm == 128) return launch_dn<128, 4>(p, s);
  if (d == 128 && p.bm == 64) return launch_dn<128, 2>(p, s);
  if (d == 64 && p.bm == 256) return launch_dn<64, 8>(p, s);
  if (d == 64 && p.bm == 128) return launch_dn<64, 4>(p, s);
  if (d == 64 && p.bm == 64) return launch_dn<64, 2>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
