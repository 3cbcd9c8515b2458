// HBM -> LDS transfers (global_load_lds_dwordx4) issued through inline asm.
//
// One instruction moves 16 bytes per lane: lane i's 16 bytes from its global
// address land at LDS byte address m0 + 16 i.  The builtin form is tracked
// by the compiler, which cannot tell apart the LDS buffers a kernel cycles
// through: it then makes the first LDS read after a transfer, and every
// workgroup barrier (whose release covers LDS writes), wait until all
// transfers in flight have landed (s_waitcnt vmcnt(0)), so a multi-stage
// pipeline degenerates to one stage.  Issued through asm the transfers are
// invisible to that analysis, and a kernel using these helpers must itself
// wait (s_waitcnt vmcnt) for the transfers that filled a buffer, then pass a
// barrier, before any wave reads that buffer; vector-memory loads complete
// in issue order, so vmcnt(n) leaves only the n most recent in flight.
// The LDS address must be wave-uniform (it is taken from the first lane).
// m0 (which the compiler may use for its own purposes and does not save
// around inline asm) is copied to a scratch SGPR, set for the transfer and
// restored in the same statement; the s_nop covers the wait state a
// transfer needs after m0 is written.
#pragma once

#include <stdint.h>

namespace dqkv {

typedef __attribute__((address_space(3))) void lds_dma_t;

// 64-bit per-lane source address.
__device__ __forceinline__ void dma16(const void* g, lds_dma_t* l) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)l);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m)
      : "memory");
}

// Wave-uniform base (moved to scalar registers) plus a 32-bit per-lane byte
// offset, so the per-tile address arithmetic stays on the scalar unit.  A
// vector-memory instruction that reads an SGPR written by a VALU instruction
// (here v_readfirstlane) needs 5 wait states in between, which the compiler
// cannot see through the asm: the leading s_nop 4 provides them.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, lds_dma_t* l) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)l);
  const uint64_t a = (uint64_t)base;
  const uint64_t su = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  uint32_t saved;
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"((const void*)su), "s"(m)
      : "memory");
}

}  // namespace dqkv
