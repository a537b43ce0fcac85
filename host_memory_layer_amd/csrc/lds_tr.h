// Direct global -> LDS loads (buffer_load_dwordx4 ... lds) issued as inline
// assembly, and the transposing LDS read.
//
// The compiler's builtin for the direct load makes every later
// ds_read_b64_tr_b16 wait for all such loads in flight (s_waitcnt
// vmcnt(0)), whatever the addresses, which defeats prefetching.  Issued as
// assembly the loads are invisible to the compiler's counters: kernels that
// use dma16 wait for them explicitly (s_waitcnt vmcnt) before reading the
// destination, as they already do for ordering across waves.  M0 holds the
// LDS destination of each load; it is set in the same statement, and no
// other instruction in these kernels reads M0.
#pragma once

#include <stdint.h>

namespace mt {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, no stride, `bytes` valid bytes
// (reads past them return zero).
__device__ inline i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const i32x4_t r = {(int)(uint32_t)a, (int)((a >> 32) & 0xFFFF), (int)bytes, 0x00020000};
  return r;
}

// Each lane loads 16 bytes at rsrc + voff + soff into LDS at lds_dst + 16 *
// lane (lds_dst wave-uniform).
__device__ inline void dma16(i32x4_t rsrc, const void* lds_dst, int voff, int soff) {
  const uint32_t m = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m), "v"(voff), "s"(rsrc),
               "s"(soff)
               : "memory", "m0");
}

// s_waitcnt vmcnt(0) as an instruction the compiler knows (expcnt and
// lgkmcnt left at their maxima, 7 and 15).  The compiler tracks only the
// global loads it issued itself; one still pending where a loop begins makes
// it wait for it inside the loop, and the hardware counter there also counts
// the direct loads of the next tile just issued, so that wait would drain the
// prefetch.  Called before such a loop, it retires the register loads ahead
// of it and no wait is left inside.
__device__ inline void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Transposing LDS read (groups of 16 lanes): output lane i, element e is
// element i%4 of the 8 bytes addressed by lane 4e + i/4 of the same group.
__device__ inline i16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

}  // namespace mt
