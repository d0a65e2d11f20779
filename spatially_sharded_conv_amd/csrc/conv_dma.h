// Operand movement helpers shared by the LDS-staged convolution kernels (gfx950).
#pragma once

#include "vaep_internal.h"

namespace vaep {
namespace dma {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(3))) unsigned short lds_u16;

constexpr unsigned kPadOffset = 0x80000000u;  // past every buffer resource (< 2 GiB, host-checked)

// Raw buffer resource over [base, base + bytes): loads past the end return zeros, which is
// how padding taps read (their offset is set past the end).
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  return u32x4_t{(unsigned)p, (unsigned)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from the buffer at voff + soff into LDS at lds + 16 * lane (lds and
// soff wave-uniform; lds goes through m0).  Written as inline assembly so that the
// compiler does not track these LDS writes: it would otherwise wait for every outstanding
// load before each LDS read, as it cannot tell the stages apart.  Completion is tracked
// by the caller with explicit vmcnt waits; its barrier asm carries a memory clobber so LDS
// reads stay after it.  The compiler's hazard checks do not look inside the asm, so it
// carries the wait states itself: 1 after the m0 write (LDS DMA reads m0), and 5 before
// the first load of a batch, whose soffset may just have been written by a VALU
// readfirstlane.
__device__ __forceinline__ void dma16(bool first, u32x4_t r, unsigned lds, unsigned voff, unsigned soff) {
  if (first)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                    "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                    "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)reinterpret_cast<unsigned long long>(
      (const lds_u16*)reinterpret_cast<const unsigned short*>(p));
}

// Workgroup id -> work id: each XCD (workgroups are dealt round-robin over 8) gets a
// contiguous run of work ids, so neighbouring tiles share rows in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int lin, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = lin & 7, i = lin >> 3;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace dma
}  // namespace vaep
