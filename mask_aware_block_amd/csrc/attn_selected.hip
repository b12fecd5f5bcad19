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

// With nsplit > 1 (few-query / decode path) workgroup (item, s) takes only
// list entries [s * per, (s + 1) * per) and writes its partial state (running
// max M, sum L, unnormalised O per head) to the workspace instead of O / LSE;
// k_selected_combine merges the splits.
template <int D, int G>
__global__ void __launch_bounds__(256) k_attn_selected(SelAttnParams p, int nsplit, float* ws) {
  constexpr int DPL = D / 64;  // output columns per lane
  __shared__ float Pl[4][CELLS][16];
  __shared__ float Al[4][16];
  __shared__ float Cm[4][16], Cl[4][16];
  __shared__ float Co[4][G][D];

  const int64_t nq = (int64_t)p.b * p.sq;
  const int64_t item = blockIdx.x / nsplit;
  const int split = (int)(blockIdx.x % nsplit);
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

  const int per = (cnt + nsplit - 1) / nsplit;
  const int e0 = split * per, e1 = min(cnt, e0 + per);
  for (int e = e0 + w; e < e1; e += 4) {
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
    // A wave that saw no entry keeps m = -FLT_MAX and l = 0: its factor is
    // exp2 of a large negative number (0), or 1 when every wave is empty, and
    // either way it adds nothing.
    float M = fmaxf(fmaxf(Cm[0][g], Cm[1][g]), fmaxf(Cm[2][g], Cm[3][g]));
    float L = 0.f, acc_o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      float f = __builtin_amdgcn_exp2f((Cm[ww][g] - M) * c);
      L += Cl[ww][g] * f;
      acc_o += Co[ww][g][d] * f;
    }
    if (nsplit > 1) {
      float* part = ws + (item * nsplit + split) * (size_t)(G * (D + 2));
      part[2 * G + g * D + d] = acc_o;
      if (d == 0) {
        part[g] = M;
        part[G + g] = L;
      }
      continue;
    }
    const int h = kvh * G + g;
    __bf16* O = (__bf16*)p.o + b * p.os[0] + h * p.os[1] + i * p.os[2];
    O[d] = (__bf16)(L > 0.f ? acc_o / L : 0.f);
    if (d == 0 && p.lse)
      p.lse[((int64_t)b * p.hq + h) * p.sq + i] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
  }
}

// Merge of the split partial states: one workgroup per (item, head), one
// thread per output column.  The combine rule is the one the split-K decode
// path of the selected-key PR uses: factors exp(m_s - M) against the largest
// partial max, with empty splits (m = -FLT_MAX, l = 0) contributing nothing.
template <int D, int G>
__global__ void __launch_bounds__(D) k_selected_combine(SelAttnParams p, int nsplit, const float* ws) {
  const int64_t item = blockIdx.x / G;
  const int g = (int)(blockIdx.x % G);
  const int d = threadIdx.x;
  const int64_t nq = (int64_t)p.b * p.sq;
  const int kvh = (int)(item / nq);
  const int64_t rem = item % nq;
  const int b = (int)(rem / p.sq);
  const int i = (int)(rem % p.sq);
  const float c = p.scale * kLog2e;
  const size_t stride = (size_t)G * (D + 2);
  const float* base = ws + item * nsplit * stride;
  // (the loops are unrolled so that eight splits' loads are in flight at once
  // rather than one latency per split)
  float M = -FLT_MAX;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[s * stride + g]);
  float L = 0.f, acc_o = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float f = __builtin_amdgcn_exp2f((base[s * stride + g] - M) * c);
    L += base[s * stride + G + g] * f;
    acc_o += base[s * stride + 2 * G + g * D + d] * f;
  }
  const int h = kvh * G + g;
  __bf16* O = (__bf16*)p.o + b * p.os[0] + h * p.os[1] + i * p.os[2];
  O[d] = (__bf16)(L > 0.f ? acc_o / L : 0.f);
  if (d == 0 && p.lse)
    p.lse[((int64_t)b * p.hq + h) * p.sq + i] = L > 0.f ? M * p.scale + logf(L) : -INFINITY;
}

template <int D, int G>
hipError_t launch_dg(const SelAttnParams& p, int nsplit, float* ws, hipStream_t s) {
  const int64_t items = (int64_t)p.hkv * p.b * p.sq;
  hipLaunchKernelGGL((k_attn_selected<D, G>), dim3((unsigned)(items * nsplit)), dim3(256), 0, s, p, nsplit,
                     ws);
  if (nsplit > 1)
    hipLaunchKernelGGL((k_selected_combine<D, G>), dim3((unsigned)(items * G)), dim3(D), 0, s, p, nsplit,
                       (const float*)ws);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const SelAttnParams& p, int nsplit, float* ws, hipStream_t s) {
  const int64_t items = (int64_t)p.hkv * p.b * p.sq;
  if (items <= 0) return hipSuccess;
  switch (p.group) {
    case 1: return launch_dg<D, 1>(p, nsplit, ws, s);
    case 2: return launch_dg<D, 2>(p, nsplit, ws, s);
    case 4: return launch_dg<D, 4>(p, nsplit, ws, s);
    case 8: return launch_dg<D, 8>(p, nsplit, ws, s);
    case 12: return launch_dg<D, 12>(p, nsplit, ws, s);
    case 16: return launch_dg<D, 16>(p, nsplit, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool selected_group_supported(int32_t group) {
  return group == 1 || group == 2 || group == 4 || group == 8 || group == 12 || group == 16;
}

size_t selected_split_ws_floats(const SelAttnParams& p, int32_t d, int32_t nsplit) {
  return (size_t)p.hkv * p.b * p.sq * nsplit * (size_t)p.group * (d + 2);
}

hipError_t launch_attn_selected_bf16(const SelAttnParams& p, int32_t d, int32_t nsplit, float* ws,
                                     hipStream_t s) {
  if (p.cells != CELLS || nsplit < 1 || (nsplit > 1 && !ws)) return hipErrorInvalidValue;
  if (d == 256) return launch_d<256>(p, nsplit, ws, s);
  if (d == 128) return launch_d<128>(p, nsplit, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
