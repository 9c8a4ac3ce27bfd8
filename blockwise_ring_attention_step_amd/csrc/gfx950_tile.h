// Device helpers shared by the bf16 D = 128 MFMA kernels (forward step and backward step) on gfx950:
// vector types, the swizzled LDS tile layout, direct HBM -> LDS copies and vmcnt waits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ra {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kD = 128;                      // head dimension of these kernels
constexpr int kRowBytes = kD * 2;            // one bf16 row (a key, value, query or output-gradient row)
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;

// LDS layout of a tile of 256-byte rows: the 16-byte chunk c of row r is stored at chunk
// c ^ swz(r), swz(r) = 4*(r%4) + (r/4)%4.  Both the 16-lane groups of row reads (16 consecutive
// rows, one chunk) and the 32-lane groups of the transpose reads (4 consecutive rows x 4 chunks)
// then hit distinct banks.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// value held by lane (lane ^ 32)
__device__ __forceinline__ float partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned lane = __lane_id();
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// s_waitcnt vmcnt(N) through the builtin, so the compiler's own wait bookkeeping sees it (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; expcnt and lgkmcnt left at
// their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte global -> LDS copy per lane: lane l's bytes at gbase + voff land at LDS address
// lds + 16 l.  Issued from inline assembly so that the compiler does not treat later LDS reads of
// other stages as possibly overlapping the copy in flight (it would otherwise wait for every
// outstanding global load before such reads).  The kernels track completion themselves: vmcnt waits
// and a workgroup barrier separate every copy from the first read of its stage.
// The LDS address goes in M0 (bound through the operand constraint, so the compiler knows the
// register's value).  The compiler cannot see the hazards of an instruction inside inline assembly,
// so the block opens with the longest wait the load's operands need: 5 wait states, for a base
// address whose SGPRs a VALU instruction has just written (v_readlane of a spilled SGPR, or
// v_readfirstlane); a load issued sooner reads the stale register, and the wrong high address bits
// fault.  It also covers the one wait state after the M0 write.
__device__ __forceinline__ void copy_to_lds16(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1" ::"v"(voff),
      "s"(gbase), "{m0}"(lds)
      : "memory");
}

// The same with 4 bytes per lane: lane l's dword at gbase + voff lands at LDS address lds + 4 l.
__device__ __forceinline__ void copy_to_lds4(const char* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_nop 4\n\t"
      "global_load_lds_dword %0, %1" ::"v"(voff),
      "s"(gbase), "{m0}"(lds)
      : "memory");
}

}  // namespace tile
}  // namespace ra
