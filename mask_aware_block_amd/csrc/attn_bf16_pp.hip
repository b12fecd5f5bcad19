// Masked attention forward on the interval encoding, bf16 inputs, fp32
// accumulation, gfx950: 256-row query tiles, two ping-pong wave groups.
//
// Same method as the 128-row kernel (compact lists of non-SKIP 64-key tiles,
// no mask on FULL tiles, element masks on PARTIAL ones, online softmax), with
// a schedule built for CDNA4's matrix cores:
//  * 8 waves, 32 query rows each, share every K/V tile, so one tile staged in
//    LDS feeds 256 rows (half the L2 -> LDS traffic per FLOP of 128 rows).
//  * Waves 0-3 (group A) and 4-7 (group B) sit on the same four SIMDs and run
//    the per-tile work in two barrier-separated phases, offset by one phase:
//        phase 0:  A: PV(j-1), QK(j)          B: softmax(j-1)
//        phase 1:  A: softmax(j)              B: PV(j-1), QK(j)
//    so one wave's exp / max / convert work overlaps the other wave's MFMA
//    work on the same SIMD.  Each wave still applies its rows' updates in
//    order (PV(j-1) before the rescale of tile j), i.e. the plain online
//    softmax.
//  * Four LDS stages: tiles j+1 and j+2 stream in (direct-to-LDS buffer loads,
//    issued two tiles ahead to cover the HBM latency) while K_j and V_{j-1}
//    are in use.  The interval columns of a tile come in the same way.
//  * Each wave classifies its own 32 x 64 block of a PARTIAL tile from the
//    staged intervals: fully masked blocks are skipped, fully visible ones run
//    without the element mask.
// Register and LDS layouts (S^T = K Q^T with the query row in the lane, P^T
// fed from registers, V^T through the transposing LDS read) are those of the
// 128-row kernel.
#include <float.h>

#include "internal.h"

namespace fmask {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int BN = 64;
constexpr int NW = 8;
constexpr int BM = 32 * NW;
constexpr int NT = 64 * NW;
constexpr int NSTAGE = 4;   // tiles j-1 (V), j (K), j+1 and j+2 (in flight)
constexpr float kLog2e = 1.4426950408889634f;

// wave-level block classification
constexpr int WB_SKIP = 0, WB_PARTIAL = 1, WB_FULL = 2;

template <int D>
struct Cfg {
  static constexpr int KCH = D / 8;
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int V_BYTES = BN * D * 2;
  static constexpr int IV_BYTES = BN * 16;
  static constexpr int STAGE = K_BYTES + V_BYTES + IV_BYTES;
  static constexpr int CHUNKS = BN * KCH;
  static constexpr int LOADS = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the workgroup");
};

template <int KCH>
__device__ inline int kswz(int key) { return key & (KCH - 1); }
template <int KCH>
__device__ inline int vswz(int key) {
  return KCH == 16 ? 4 * (key & 3) : 4 * ((key >> 1) & 1);
}

__device__ inline int logical_item(int gsz) {
  int p = blockIdx.x;
  int xcd = p % kXcds, k = p / kXcds;
  return ((k / gsz) * kXcds + xcd) * gsz + (k % gsz);
}

__device__ inline int overlap(int r0, int r1, int a, int b) {
  int lo = max(r0, a), hi = min(r1, b);
  return hi > lo ? hi - lo : 0;
}

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));

// Buffer resource (base, range in bytes), raw, range-checked; kept in SGPRs.
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// Direct-to-LDS buffer loads: lane i's data lands at lds + i * size.  Issued
// as inline assembly so the compiler does not order every later LDS read
// behind them; the kernel waits for them itself (vmcnt) before the barrier
// that publishes a stage.  No VGPR is written.
__device__ inline void dma16(rsrc_t r, int voff, const void* lds) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(uintptr_t)(LDS_AS const void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ inline void dma4(rsrc_t r, int voff, const void* lds) {
  const int m0 = __builtin_amdgcn_readfirstlane((int)(uintptr_t)(LDS_AS const void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
// Workgroup barrier without the memory fence of __syncthreads(): stage
// hand-over is ordered by explicit waits (vmcnt for the loads; every LDS read
// of a phase is consumed by that phase's MFMAs before the barrier).
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int D>
__global__ void __launch_bounds__(NT, 1) k_attn_pp_bf16(TileAttnParams p, int gsz) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * C::STAGE];

  const int l = logical_item(gsz);
  if (l >= p.n_items) return;
  // decode the work item (tile row of the order, then the (b, h) it covers)
  const int row = p.order[l / p.expand];
  const int e = l % p.expand;
  const int qt = row % p.nqt;
  const int mh = (row / p.nqt) % p.mh;
  const int mb = row / (p.nqt * p.mh);
  int b, h;
  if (p.mb == 1 && p.mh == 1) { b = e / p.hq; h = e % p.hq; }
  else if (p.mb == 1) { b = e; h = mh; }
  else if (p.mh == 1) { b = mb; h = e; }
  else { b = mb; h = mh; }
  const int kvh = h / p.group;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept scalar
  const int lane = tid & 63;
  const int grp = w >> 2;  // 0: group A, 1: group B
  const int half = lane >> 5, l32 = lane & 31;
  const int q0 = qt * BM;
  const int r0 = q0 + w * 32;
  const int qrow = r0 + l32;
  const bool wave_live = r0 < p.sq;

  const __bf16* Q = (const __bf16*)p.q + b * p.qs[0] + h * p.qs[1];
  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];
  const int32_t* list = p.list + (int64_t)row * p.nkt;
  const int cnt = p.count[row];
  const int64_t ks2 = p.ks[2], vs2 = p.vs[2];
  const int32_t* ivcol = p.iv + ((size_t)mb * p.mh + mh) * 4 * (size_t)p.skv;

  // The ragged last key tile reads rows past the end as zeros; clear LDS once
  // so those rows never hold stale NaN bits before the first load lands.
  if (cnt > 0 && (list[cnt - 1] & 0x7fffffff) == p.nkt - 1 && p.skv % BN != 0)
    for (int i = tid; i < NSTAGE * C::STAGE / 16; i += NT) ((i32x4*)smem)[i] = i32x4{0, 0, 0, 0};

  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qrow < p.sq) qf[t] = *(const bf16x8*)(Q + qrow * p.qs[2] + 16 * t + 8 * half);
    else qf[t] = bf16x8{};
  }

  // Q must be in registers before any tile load goes out: the loads below are
  // invisible to the compiler's wait counting, so nothing tracked may be left
  // pending across them.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -FLT_MAX, l_run = 0.f;
  const float c = p.scale * kLog2e;

  const rsrc_t krs = make_rsrc(K, ((int64_t)(p.skv - 1) * ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(V, ((int64_t)(p.skv - 1) * vs2 + D) * 2);

  int kgo[C::LOADS], vgo[C::LOADS];
#pragma unroll
  for (int n = 0; n < C::LOADS; ++n) {
    const int P = (w * C::LOADS + n) * 64 + lane;
    const int key = P / C::KCH, pc = P % C::KCH;
    kgo[n] = (int)(key * ks2 * 2 + ((pc ^ kswz<C::KCH>(key)) * 16));
    vgo[n] = (int)(key * vs2 * 2 + ((pc ^ vswz<C::KCH>(key)) * 16));
  }
  const int kstep = (int)(BN * ks2 * 2), vstep = (int)(BN * vs2 * 2);

  const int tg = lane >> 4, tr = (lane >> 2) & 3, tc4 = lane & 3;
  const int vrow_l = 4 * (tg >> 1) + tr;
  int vofs[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int ch = 4 * db + 2 * (tg & 1) + (tc4 >> 1);
    vofs[db] = vrow_l * (D * 2) + ((ch ^ vswz<C::KCH>(vrow_l)) * 16) + (tc4 & 1) * 8;
  }

  // Interval columns of a tile: wave f < 4 loads field f (UTS, UTE, LTS, LTE)
  // of the tile's 64 keys, one dword per lane, giving an LDS block [4][64]
  // int32.  Keys past skv read garbage or zero and are masked explicitly.
  const rsrc_t irs = make_rsrc(ivcol, 4 * (int64_t)p.skv * 4);
  const int igo = (w & 3) * p.skv * 4 + lane * 4;

  // Issue the direct-to-LDS loads of tile kt into stage buf.
  auto issue_tile = [&](int kt, int buf) {
    char* kb = smem + buf * C::STAGE;
    char* vb = kb + C::K_BYTES;
    const int kb0 = kt * kstep, vb0 = kt * vstep;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) dma16(krs, kgo[n] + kb0, kb + (w * C::LOADS + n) * 1024);
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) dma16(vrs, vgo[n] + vb0, vb + (w * C::LOADS + n) * 1024);
    if (w < 4) dma4(irs, igo + kt * BN * 4, vb + C::V_BYTES + w * 256);
  };

  // Per-wave state: S of the tile being scored, P of the tile awaiting PV.
  f32x16 s[2];
  bf16x8 pf[4];
  int st_s = WB_SKIP, st_p = WB_SKIP;  // wave-block class of the tile in s / in pf

  // Score tile kt (stage buf) for this wave's rows: class, S^T = K Q^T, mask.
  auto qk = [&](int buf, int kt, bool tile_full) {
    const char* kb = smem + buf * C::STAGE;
    const char* ivb = kb + C::K_BYTES + C::V_BYTES;
    const int32_t* ivf = (const int32_t*)ivb;  // [4][64]: UTS, UTE, LTS, LTE
    const int kvalid = p.skv - kt * BN;         // keys of this tile that exist
    int st = WB_FULL;
    if (!wave_live) {
      st = WB_SKIP;
    } else if (!tile_full || kvalid < BN) {
      // lane k checks key column k over the wave's 32 rows
      const int r1 = r0 + 32;
      int mc = overlap(r0, r1, ivf[lane], ivf[64 + lane]) + overlap(r0, r1, ivf[128 + lane], ivf[192 + lane]);
      if (lane >= kvalid) mc = 32;
      // rows past the end count as masked so a wave straddling sq can still skip
      if (r1 > p.sq) mc = min(32, mc + (r1 - p.sq));
      const bool all_m = __all(mc == 32), none_m = __all(mc == 0);
      st = all_m ? WB_SKIP : (none_m ? WB_FULL : WB_PARTIAL);
    }
    st_s = st;
    if (st == WB_SKIP) return;
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
    if (st == WB_PARTIAL) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int k0 = kh * 32 + 8 * rg + 4 * half;  // 4 consecutive keys k0 .. k0 + 3
          const i32x4 uts = *(const i32x4*)(ivf + k0), ute = *(const i32x4*)(ivf + 64 + k0);
          const i32x4 lts = *(const i32x4*)(ivf + 128 + k0), lte = *(const i32x4*)(ivf + 192 + k0);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const bool masked = (qrow >= uts[r4] && qrow < ute[r4]) || (qrow >= lts[r4] && qrow < lte[r4]) ||
                                k0 + r4 >= kvalid;
            if (masked) s[kh][rg * 4 + r4] = -INFINITY;
          }
        }
    }
  };

  // Online softmax of the scored tile into pf (bf16 P^T), rescaling O when the
  // running max moves by more than 8 in exp2 units.
  auto softmax = [&]() {
    st_p = st_s;
    if (st_s == WB_SKIP) return;
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
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        f32x8 pv;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][8 * tp + j], c, mneg));
        pf[kh * 2 + tp] = __builtin_convertvector(pv, bf16x8);
      }
    const bf16x2 one2 = bf16x2{(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x2 pr = bf16x2{pf[ks][2 * j], pf[ks][2 * j + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_run, false);
      }
  };

  // O^T += V^T P^T with V from stage buf.
  auto pv = [&](int buf) {
    if (st_p == WB_SKIP) return;
    const char* vb = smem + buf * C::STAGE + C::K_BYTES;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const char* a0 = vb + vofs[db] + (16 * ks) * (D * 2);
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)a0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(a0 + 8 * (D * 2)));
        bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
      }
  };

  __syncthreads();  // LDS clear (if any) before the first loads land
  // Prologue: tiles 0 and 1 into stages 0 and 1.  List entries are read two
  // tiles ahead of their use.
  // (scalar loads: their waits use lgkmcnt and never wait for tile data)
  int e0 = 0, e1 = 0, e2 = 0;  // entries of tiles j, j+1, j+2
  if (cnt > 0) e0 = list[0];
  if (cnt > 1) e1 = list[1];
  if (cnt > 2) e2 = list[2];
  if (cnt > 0) issue_tile(e0 & 0x7fffffff, 0);
  if (cnt > 1) issue_tile(e1 & 0x7fffffff, 1);
  // tile 0 must be in LDS; tile 1 may still be in flight (vmcnt(n_issue))
  if (cnt > 1 && w < 4) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::LOADS + 1));
  else if (cnt > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::LOADS));
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // Iteration j scores tile j (stage j % 4) and multiplies P of tile j-1 into
  // V_{j-1} (stage (j-1) % 4); tile j+2 starts streaming into stage (j+2) % 4.
  for (int j = 0; j <= cnt; ++j) {
    const bool have_j = j < cnt, have_prev = j > 0;
    const bool tile_full = (e0 & (int)FMASK_LIST_FULL_BIT) != 0;
    const int kt = e0 & 0x7fffffff;
    const int buf_j = j & (NSTAGE - 1), buf_prev = (j - 1) & (NSTAGE - 1);
    int e3 = 0;
    const bool issue = j + 2 < cnt;
    if (issue) {
      e3 = list[min(j + 3, cnt - 1)];
      issue_tile(e2 & 0x7fffffff, (j + 2) & (NSTAGE - 1));
    }
    // phase 0
    SCHED_FENCE();
    if (grp == 0) {
      if (have_prev) pv(buf_prev);
      if (have_j) qk(buf_j, kt, tile_full);
    } else {
      if (have_prev) softmax();
    }
    SCHED_FENCE();
    barrier();
    SCHED_FENCE();
    // phase 1
    if (grp == 0) {
      if (have_j) softmax();
    } else {
      if (have_prev) pv(buf_prev);
      if (have_j) qk(buf_j, kt, tile_full);
    }
    SCHED_FENCE();
    // tile j+1 must have landed; only tile j+2's loads may still be in flight
    if (issue && w < 4) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::LOADS + 1));
    else if (issue) __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::LOADS));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    barrier();
    SCHED_FENCE();
    e0 = e1;
    e1 = e2;
    e2 = e3;
  }

  // Epilogue: O = O / l, zero rows for l = 0, LSE in natural log.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.sq) {
    __bf16* O = (__bf16*)p.o + b * p.os[0] + h * p.os[1] + qrow * p.os[2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = db * 32 + 8 * rg + 4 * half;
        f32x4 x = f32x4{acc[db][4 * rg], acc[db][4 * rg + 1], acc[db][4 * rg + 2],
                        acc[db][4 * rg + 3]} * inv;
        *(bf16x4*)(O + d0) = __builtin_convertvector(x, bf16x4);
      }
    if (p.lse && half == 0) {
      float lse = l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
      p.lse[((int64_t)b * p.hq + h) * p.sq + qrow] = lse;
    }
  }
#endif
}

}  // namespace

hipError_t launch_attn_pp_bf16(const TileAttnParams& p, int32_t d, hipStream_t s) {
  if (p.bn != BN || p.bm != BM || p.kind != FMASK_ENC_INTERVALS) return hipErrorInvalidValue;
  if (p.n_items <= 0) return hipSuccess;
  int gsz = (p.mh == 1) ? p.group : 1;
  int64_t unit = (int64_t)kXcds * gsz;
  int64_t npad = (p.n_items + unit - 1) / unit * unit;
  if (d == 128)
    hipLaunchKernelGGL(k_attn_pp_bf16<128>, dim3((unsigned)npad), dim3(NT), 0, s, p, gsz);
  else if (d == 64)
    hipLaunchKernelGGL(k_attn_pp_bf16<64>, dim3((unsigned)npad), dim3(NT), 0, s, p, gsz);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fmask
