// Masked attention forward, fp32 inputs and arithmetic (VALU), 64 x 64 tiles.
//
// Same method as the bf16 MFMA kernel (walk the compact list of non-SKIP key
// tiles, no mask on FULL tiles, element masks on PARTIAL ones, online softmax)
// but in plain fp32 so that results stay within 1e-5 of a float64 reference.
// 256 threads per 64-row query tile: thread t owns row t / 4 and scores keys
// 16 (t % 4) .. +15 of every key tile, then accumulates output columns
// (t % 4) * d / 4 .. +d/4 - 1 over all 64 keys of the tile.
#include <float.h>

#include "internal.h"

namespace fmask {
namespace {

constexpr int BM = 64, BN = 64;

template <int D, int KIND>
__global__ void __launch_bounds__(256) k_attn_tile_f32(TileAttnParams p) {
  __shared__ float Qs[BM][D];
  __shared__ float Ks[BN][D + 1];
  __shared__ float Vs[BN][D];
  __shared__ float Ps[BM][BN + 1];
  __shared__ int32_t Iv[BN][4];

  const int l = blockIdx.x;
  if (l >= p.n_items) return;
  int row_idx = p.order[l / p.expand];
  int e = l % p.expand;
  int qt = row_idx % p.nqt;
  int mh = (row_idx / p.nqt) % p.mh;
  int mb = row_idx / (p.nqt * p.mh);
  int b, h;
  if (p.mb == 1 && p.mh == 1) { b = e / p.hq; h = e % p.hq; }
  else if (p.mb == 1) { b = e; h = mh; }
  else if (p.mh == 1) { b = mb; h = e; }
  else { b = mb; h = mh; }
  const int kvh = h / p.group;

  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int q0 = qt * BM;
  const int qrow = q0 + r;
  const float* Q = (const float*)p.q + b * p.qs[0] + h * p.qs[1];
  const float* K = (const float*)p.k + b * p.ks[0] + kvh * p.ks[1];
  const float* V = (const float*)p.v + b * p.vs[0] + kvh * p.vs[1];
  const int32_t* list = p.list + (int64_t)row_idx * p.nkt;
  const int cnt = p.count[row_idx];

  for (int i = tid; i < BM * D; i += 256) {
    int rr = i / D, d = i % D;
    Qs[rr][d] = (q0 + rr < p.sq) ? Q[(q0 + rr) * p.qs[2] + d] : 0.f;
  }

  constexpr int DP = D / 4;
  float o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) o[i] = 0.f;
  float m_run = -FLT_MAX, l_run = 0.f;
  const size_t mbase = (size_t)mb * p.mh + mh;

  for (int it = 0; it < cnt; ++it) {
    const uint32_t ent = (uint32_t)list[it];
    const int kt = (int)(ent & 0x7fffffffu);
    const bool full = (ent & FMASK_LIST_FULL_BIT) != 0;
    const int key0 = kt * BN;
    __syncthreads();  // previous tile fully consumed
    for (int i = tid; i < BN * D; i += 256) {
      int kk = i / D, d = i % D;
      bool ok = key0 + kk < p.skv;
      Ks[kk][d] = ok ? K[(key0 + kk) * p.ks[2] + d] : 0.f;
      Vs[kk][d] = ok ? V[(key0 + kk) * p.vs[2] + d] : 0.f;
    }
    if (KIND == FMASK_ENC_INTERVALS && tid < BN) {
      int key = key0 + tid;
      if (key < p.skv) {
        const int32_t* col = p.iv + mbase * 4 * (size_t)p.skv;
        Iv[tid][0] = col[key];
        Iv[tid][1] = col[p.skv + key];
        Iv[tid][2] = col[2 * (size_t)p.skv + key];
        Iv[tid][3] = col[3 * (size_t)p.skv + key];
      } else {
        Iv[tid][0] = 0; Iv[tid][1] = 0x7fffffff; Iv[tid][2] = 0; Iv[tid][3] = 0;
      }
    }
    __syncthreads();

    const bool ragged = key0 + BN > p.skv;
    bool need_mask = !full || ragged;
    uint64_t word = ~0ull;
    if (KIND == FMASK_ENC_BITMAP) {
      size_t bidx = (mbase * p.nbq + qt) * p.nbk + kt;
      uint8_t st = p.bstate[bidx];
      if (st == FMASK_PARTIAL) {
        word = p.bbits[(int64_t)p.bindex[bidx] * kBlk + r];
        need_mask = true;
      } else if (st == FMASK_SKIP) {
        word = 0;
        need_mask = true;
      } else {
        int valid = p.skv - key0;
        word = valid >= 64 ? ~0ull : ((1ull << valid) - 1ull);
      }
    }

    float s[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int j = part * 16 + jj;
      float acc = 0.f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(Qs[r][d], Ks[j][d], acc);
      acc *= p.scale;
      if (need_mask) {
        bool masked;
        if (KIND == FMASK_ENC_INTERVALS)
          masked = (qrow >= Iv[j][0] && qrow < Iv[j][1]) || (qrow >= Iv[j][2] && qrow < Iv[j][3]);
        else
          masked = ((word >> j) & 1ull) == 0;
        if (masked) acc = -INFINITY;
      }
      s[jj] = acc;
      mloc = fmaxf(mloc, acc);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 1));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 2));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = expf(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      float pj = expf(s[jj] - m_new);
      lsum += pj;
      Ps[r][part * 16 + jj] = pj;
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < DP; ++i) o[i] *= alpha;
    __syncthreads();
    for (int j = 0; j < BN; ++j) {
      const float pj = Ps[r][j];
#pragma unroll
      for (int i = 0; i < DP; ++i) o[i] = __builtin_fmaf(pj, Vs[j][part * DP + i], o[i]);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 1);
  l_tot = l_tot + __shfl_xor(l_tot, 2);
  if (qrow < p.sq) {
    float* O = (float*)p.o + b * p.os[0] + h * p.os[1] + qrow * p.os[2] + part * DP;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int i = 0; i < DP; ++i) O[i] = o[i] * inv;
    if (p.lse && part == 0)
      p.lse[((int64_t)b * p.hq + h) * p.sq + qrow] = l_tot > 0.f ? m_run + logf(l_tot) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const TileAttnParams& p, hipStream_t s) {
  if (p.n_items <= 0) return hipSuccess;
  if (p.kind == FMASK_ENC_INTERVALS)
    hipLaunchKernelGGL((k_attn_tile_f32<D, FMASK_ENC_INTERVALS>), dim3(p.n_items), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_attn_tile_f32<D, FMASK_ENC_BITMAP>), dim3(p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_tile_f32(const TileAttnParams& p, int32_t d, hipStream_t s) {
  if (p.bm != BM || p.bn != BN) return hipErrorInvalidValue;
  if (d == 64) return launch_d<64>(p, s);
  if (d == 128) return launch_d<128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fmask
