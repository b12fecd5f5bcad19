// Selected-key attention forward (bf16, fp32 accumulation).
//
// Visibility is a per-query list of K/V blocks of 32 cells; there is no dense
// mask and no causal term (llama.cpp selected-key PR: the list is the only
// source of visibility, invalid and duplicate entries are skipped; the lists
// arrive here already canonical: valid, distinct, ascending).
//
// One workgroup per (K/V head, batch, query): its 4 waves take every 4th block
// of the query's list.  Per block a wave
//   * scores the block's 32 keys against the group's query heads with
//     v_mfma_f32_16x16x32_bf16 (A = K rows straight from global memory, B =
//     Q^T of the group's heads in registers, columns beyond the group idle);
//   * runs the online softmax per head (exp2 domain, max from -FLT_MAX);
//   * accumulates P V on the VALU, each lane owning d / 64 output columns of
//     every head, reading whole V rows coalesced.
// The waves' partial (m, l, O) are merged in LDS at the end, the same combine
// as a split-K reduce; an empty list yields O = 0 and LSE = -inf.
// Work items are ordered K/V-head-major so one head's K/V (a few hundred MiB
// at 128K context) is what the chip's caches hold at a time.
#include <float.h>

#include "internal.h"

namespace fmask {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int CELLS = 32;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ inline float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int D, int G>
__global__ void __launch_bounds__(256) k_attn_selected(SelAttnParams p) {
  constexpr int DPL = D / 64;  // output columns per lane
  __shared__ float Pl[4][CELLS][16];
  __shared__ float Al[4][16];
  __shared__ float Cm[4][16], Cl[4][16];
  __shared__ float Co[4][G][D];

  const int64_t nq = (int64_t)p.b * p.sq;
  const int64_t item = blockIdx.x;
  const int kvh = (int)(item / nq);
  const int64_t rem = item % nq;
  const int b = (int)(rem / p.sq);
  const int i = (int)(rem % p.sq);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 15, quad = lane >> 4;
  const int mb = p.mb > 1 ? b : 0;
  const int32_t* lst = p.list + ((int64_t)mb * p.sq + i) * p.n;
  const int cnt = p.count[(int64_t)mb * p.sq + i];
  const float c = p.scale * kLog2e;

  // Q^T (B operand): lane holds head kvh*G + col, d = 32 t + 8 quad + 0..7.
  bf16x8 qf[D / 32];
  {
    const __bf16* Q = (const __bf16*)p.q + b * p.qs[0] + i * p.qs[2];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      if (col < G) qf[t] = *(const bf16x8*)(Q + (kvh * G + col) * p.qs[1] + 32 * t + 8 * quad);
      else qf[t] = bf16x8{};
    }
  }
  const __bf16* K = (const __bf16*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const __bf16* V = (const __bf16*)p.v + b * p.vs[0] + kvh * p.vs[1];

  float acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[g][j] = 0.f;
  float m_run = -FLT_MAX, l_run = 0.f;  // per column (head) lane

  for (int e = w; e < cnt; e += 4) {
    const int64_t kbase = (int64_t)lst[e] * CELLS;
    // Gather: K rows as MFMA A operands, V rows for the VALU accumulation.
    bf16x8 ka[2][D / 32];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      int64_t key = kbase + kh * 16 + col;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        if (key < p.skv) ka[kh][t] = *(const bf16x8*)(K + key * p.ks[2] + 32 * t + 8 * quad);
        else ka[kh][t] = bf16x8{};
      }
    }
    u32x2 vr[CELLS][DPL / 4 > 0 ? DPL / 4 : 1];
    uint32_t vr1[CELLS];
#pragma unroll
    for (int k = 0; k < CELLS; ++k) {
      int64_t key = kbase + k;
      if constexpr (DPL == 4) {
        vr[k][0] = key < p.skv ? *(const u32x2*)(V + key * p.vs[2] + lane * DPL) : u32x2{0, 0};
      } else {
        vr1[k] = key < p.skv ? *(const uint32_t*)(V + key * p.vs[2] + lane * DPL) : 0u;
      }
    }
    // S^T[key][head] for keys kh*16 + 4 quad + r.
    f32x4 s[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      s[kh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        s[kh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kh][t], qf[t], s[kh], 0, 0, 0);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (kbase + kh * 16 + 4 * quad + r >= p.skv) s[kh][r] = -INFINITY;
        mloc = fmaxf(mloc, s[kh][r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    const float mneg = -m_new * c;
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kh][r], c, mneg));
        lsum += pv;
        if (col < G) Pl[w][kh * 16 + 4 * quad + r][col] = pv;
      }
    l_run = l_run * alpha + lsum;
    if (quad == 0 && col < G) Al[w][col] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float a = Al[w][g];
#pragma unroll
      for (int j = 0; j < DPL; ++j) acc[g][j] *= a;
    }
#pragma unroll
    for (int k = 0; k < CELLS; ++k) {
      float vv[DPL];
      if constexpr (DPL == 4) {
        vv[0] = bf_lo(vr[k][0][0]); vv[1] = bf_hi(vr[k][0][0]);
        vv[2] = bf_lo(vr[k][0][1]); vv[3] = bf_hi(vr[k][0][1]);
      } else {
        vv[0] = bf_lo(vr1[k]); vv[1] = bf_hi(vr1[k]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pg = Pl[w][k][g];
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[g][j] = __builtin_fmaf(pg, vv[j], acc[g][j]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Merge the four waves' partial states.
  float l_col = l_run + __shfl_xor(l_run, 16);
  l_col = l_col + __shfl_xor(l_col, 32);
  if (quad == 0 && col < G) {
    Cm[w][col] = m_run;
    Cl[w][col] = l_col;
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < DPL; ++j) Co[w][g][lane * DPL + j] = acc[g][j];
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, d = x % D;
    float M = fmaxf(fmaxf(Cm[0][g], Cm[1][g]), fmaxf(Cm[2][g], Cm[3][g]));
    float L = 0.f, acc_o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      float f = __builtin_amdgcn_exp2f((Cm[ww][g] - M) * c);
      L += Cl[ww][g] * f;
      acc_o += Co[ww][g][d] * f;
    }
    const int h = kvh * G + g;
    __bf16* O = (__bf16*)p.o + b * p.os[0] + h * p.os[1] + i * p.os[2];
    O[d] = (__bf16)(L > 0.f ? acc_o / L : 0.f);
    if (d == 0 && p.lse)
      p.lse[((int64_t)b * p.hq + h) * p.sq + i] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const SelAttnParams& p, hipStream_t s) {
  int64_t items = (int64_t)p.hkv * p.b * p.sq;
  if (items <= 0) return hipSuccess;
  dim3 grid((unsigned)items), block(256);
  switch (p.group) {
    case 1: hipLaunchKernelGGL((k_attn_selected<D, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_attn_selected<D, 2>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_attn_selected<D, 4>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((k_attn_selected<D, 8>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((k_attn_selected<D, 16>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_selected_bf16(const SelAttnParams& p, int32_t d, hipStream_t s) {
  if (p.cells != CELLS) return hipErrorInvalidValue;
  if (d == 256) return launch_d<256>(p, s);
  if (d == 128) return launch_d<128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
