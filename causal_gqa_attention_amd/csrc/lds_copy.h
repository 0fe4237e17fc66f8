// LDS helpers shared by the MFMA kernels (gfx950): LDS-typed pointers, wait counts and
// the direct global -> LDS copy (buffer_load_dwordx4 ... lds) with a per-tile range check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xattn_device.h"

namespace xattn {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) const bf16x8 lds_cbf16x8_t;
typedef __attribute__((address_space(3))) const char lds_cchar_t;
using lptr = lds_cchar_t*;  // LDS operand tiles are read through LDS-typed pointers

// LDS address of a generic pointer into LDS: its low 32 bits.  Taken once per buffer, so
// the offsets added after it fold into the LDS instructions, and without the null test
// that an address-space cast of a generic pointer carries.
__device__ __forceinline__ lptr to_lds(const char* p) {
  return (lptr)(uintptr_t)(uint32_t)(uintptr_t)p;
}
typedef __attribute__((ext_vector_type(4))) int i32x4;

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void lds_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Direct global -> LDS copies (gfx950 global_load_lds): lane l's bytes land at the
// wave-uniform LDS address dst + size * l.  They are written as inline assembly so that the
// compiler does not see an LDS write in flight: it would otherwise make every later
// transposing LDS read wait for all outstanding loads, prefetches included.  Callers order
// the copies against LDS reads themselves, with vmcnt waits and barriers.  M0 (the LDS
// destination) is saved and restored around the copy; one wait state separates its write
// from the load that reads it.
// PER consecutive 1 KiB wave copies into dst, dst + 1 KiB, ...: lane l of copy j reads
// byte voff[j] of a raw buffer of nbytes bytes at gbase (buffer_load_dwordx4 ... lds).  The
// buffer's range check turns reads at or past nbytes into zeros, so tiles that run past the
// sequence end need no clamping.  M0 is saved once and stepped between the copies.
template <int PER>
__device__ __forceinline__ void dma16_rows(void* dst, const char* gbase, uint32_t nbytes,
                                           const uint32_t (&voff)[PER]) {
  // every operand is wave-uniform; readfirstlane keeps them in scalar registers
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  const uint64_t ga = (uint64_t)(uintptr_t)gbase;
  i32x4 rsrc;  // base, stride 0, nbytes, raw 32-bit format
  rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)ga);
  rsrc[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(ga >> 32) & 0xFFFFu));
  rsrc[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  rsrc[3] = 0x00020000;
  uint32_t saved;
#define XATTN_LD(i) "buffer_load_dwordx4 %[o" #i "], %[r], 0 offen lds\n\t"
#define XATTN_STEP "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\t"
#define XATTN_HEAD "s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[m]\n\ts_nop 0\n\t"
#define XATTN_TAIL "s_mov_b32 m0, %[sv]"
  if constexpr (PER == 1) {
    asm volatile(XATTN_HEAD XATTN_LD(0) XATTN_TAIL
                 : [sv] "=&s"(saved) : [m] "s"(m0v), [r] "s"(rsrc), [o0] "v"(voff[0])
                 : "memory", "scc");
  } else if constexpr (PER == 2) {
    asm volatile(XATTN_HEAD XATTN_LD(0) XATTN_STEP XATTN_LD(1) XATTN_TAIL
                 : [sv] "=&s"(saved) : [m] "s"(m0v), [r] "s"(rsrc), [o0] "v"(voff[0]),
                   [o1] "v"(voff[1])
                 : "memory", "scc");
  } else if constexpr (PER == 4) {
    asm volatile(XATTN_HEAD XATTN_LD(0) XATTN_STEP XATTN_LD(1) XATTN_STEP XATTN_LD(2)
                     XATTN_STEP XATTN_LD(3) XATTN_TAIL
                 : [sv] "=&s"(saved) : [m] "s"(m0v), [r] "s"(rsrc), [o0] "v"(voff[0]),
                   [o1] "v"(voff[1]), [o2] "v"(voff[2]), [o3] "v"(voff[3])
                 : "memory", "scc");
  } else {
    static_assert(PER == 8, "1, 2, 4 or 8 copies");
    asm volatile(XATTN_HEAD XATTN_LD(0) XATTN_STEP XATTN_LD(1) XATTN_STEP XATTN_LD(2)
                     XATTN_STEP XATTN_LD(3) XATTN_STEP XATTN_LD(4) XATTN_STEP XATTN_LD(5)
                         XATTN_STEP XATTN_LD(6) XATTN_STEP XATTN_LD(7) XATTN_TAIL
                 : [sv] "=&s"(saved) : [m] "s"(m0v), [r] "s"(rsrc), [o0] "v"(voff[0]),
                   [o1] "v"(voff[1]), [o2] "v"(voff[2]), [o3] "v"(voff[3]), [o4] "v"(voff[4]),
                   [o5] "v"(voff[5]), [o6] "v"(voff[6]), [o7] "v"(voff[7])
                 : "memory", "scc");
  }
#undef XATTN_LD
#undef XATTN_STEP
#undef XATTN_HEAD
#undef XATTN_TAIL
}
}  // namespace xattn
