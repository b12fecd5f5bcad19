// Device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmask {

#define FMASK_LDS_AS __attribute__((address_space(3)))

typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): 32-bit offsets, loads past
// the range return zero.  All four words are scalar.
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

__device__ inline int lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((int)(uintptr_t)(FMASK_LDS_AS const void*)p);
}

// Direct-to-LDS buffer loads: lane i's 16 (or 4) bytes land at lds + 16 i
// (4 i).  Written as inline assembly with no register output, so the
// compiler's wait counting does not see them: it neither orders later LDS
// reads behind them nor drains them when waiting for an ordinary load.  The
// kernels make the data visible themselves (vmcnt wait, then a barrier).
// `lds` is the LDS byte address (see lds_addr), wave-uniform.  A scalar write
// of M0 needs one wait state before a memory instruction with the LDS bit
// reads it (AMD CDNA4 ISA reference guide, "Manually Inserted Wait States
// (NOPs)": S_MOV to M0 followed by an LDS-DMA load, 1 wait state); the
// compiler pads only the code it generates, not inline assembly, hence the
// s_nop between the two.  Without it the load may use the previous M0 and put
// its data into the previous load's destination.
__device__ inline void dma16(rsrc_t r, int voff, int lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
// Same, with a wave-uniform byte offset added through the scalar offset field.
__device__ inline void dma16s(rsrc_t r, int voff, int soff, int lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
__device__ inline void dma4(rsrc_t r, int voff, int lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}

// s_waitcnt encodings (gfx9): vmcnt in bits 3:0 (and 15:14), expcnt 6:4,
// lgkmcnt 11:8.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
__device__ inline void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }  // vmcnt(0) lgkmcnt(0)

// Workgroup barrier without __syncthreads()'s fence: the caller has already
// waited for what the barrier publishes.
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Scalar load of one int with its wait in the same block (never left pending).
__device__ inline int sload_wait(const int32_t* p) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// One byte of a device array by a scalar load of the aligned 4-byte word that
// holds it (wave-uniform address).  The word never leaves the byte's own
// aligned 4 bytes, so any base alignment is fine.
__device__ inline int sload_byte(const uint8_t* p) {
  const uintptr_t a = (uintptr_t)p;
  const int w = sload_wait((const int32_t*)(a & ~(uintptr_t)3));
  return (w >> (8 * (int)(a & 3))) & 0xff;
}

}  // namespace fmask
