// LDS staging helpers shared by the gfx950 matrix-core kernels of libptb:
// buffer resources, global -> LDS DMA, explicit wait counts, and the
// transposing fragment read of tiles stored outer-contiguous.
#pragma once

#include "device_common.h"

namespace ptb {

constexpr int kOutOfRange = static_cast<int>(0x80000000u);  // beyond any operand (< 2^31 bytes)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer resource over one operand segment: reads at or beyond `bytes` return
// zero (ragged row counts and the k tail need no branches).
__device__ __forceinline__ i32x4 make_desc(const u16* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  d[1] = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));
  d[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  d[3] = 0x00020000;
  return d;
}

// 16 bytes per lane from global memory (descriptor, per-lane byte offset voff
// plus wave-uniform byte offset soff) straight to LDS at byte address
// lds_addr + 16 * lane.  Written as inline assembly so that the compiler does
// not treat it as an LDS store (it would then wait for every outstanding load
// before any later LDS read); the kernel orders it with explicit vmcnt waits
// and barriers.  m0 is written here and read only by the load after it.
// Wait states: the compiler does not apply its hazard rules to operands of
// inline assembly, and the scalar operands here typically come from
// v_readfirstlane just before.  A vector-memory instruction reading an SGPR
// written by a VALU instruction needs 5 wait states, and one reading m0 after
// s_mov needs 1; s_mov + s_nop 3 give 5 before the load.  Without them the
// load can see a stale descriptor or offset: wrong data, or, when the range
// check of an out-of-range load is lost with the descriptor, a memory fault.
__device__ __forceinline__ void lds_dma16(i32x4 desc, uint32_t lds_addr, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  i32x4 d;  // wave-uniform by construction; keep it in scalar registers
#pragma unroll
  for (int k = 0; k < 4; ++k) d[k] = __builtin_amdgcn_readfirstlane(desc[k]);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 3\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_addr))), "v"(voff),
                 "s"(d), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
#endif
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
#else
  return 0;
#endif
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this
// wave outstanding and all of its LDS reads returned (expcnt not waited on).
// The barriers that follow it rely on both: gfx950 does not wait for
// outstanding memory operations at s_barrier.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the 4
// u16 at its address; lane i receives element i % 4 of the values supplied by
// lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.
__device__ __forceinline__ v4s lds_read_tr16(const u16* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
#else
  return v4s{};
#endif
}

// Tiles stored outer-contiguous as [64-wide outer block][KR k][64 outer]
// (128-byte rows): chunk c of k-row kk sits at chunk slot c ^ oswz(kk).
__device__ __forceinline__ int oswz(int kk) { return (kk & 2) << 1; }

// MFMA operand fragment, read transposed from such a tile: outer indices
// [rb, rb + 32), k-step ks (16 k); lane l gets X[rb + l % 32][16 ks + 8 (l / 32)
// .. +7].  Each 16-lane group reads 4 k-rows x 16 outer indices (4 u16 per
// lane), and the transposing read hands lane i the 4 k-values of its index.
template <int KR>
__device__ __forceinline__ bf16x8 frag_outer(const u16* tile, int rb, int ks, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int m = rb + 16 * (q & 1) + 4 * (j & 3);
  v4s h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int kk = ks * 16 + 8 * (q >> 1) + 4 * hh + (j >> 2);
    h[hh] = lds_read_tr16(tile + (m >> 6) * (KR * 64) + kk * 64 + ((((m >> 3) & 7) ^ oswz(kk)) << 3) +
                          (m & 7));
  }
  uint4 u;
  u.x = static_cast<uint16_t>(h[0][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[0][1])) << 16);
  u.y = static_cast<uint16_t>(h[0][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[0][3])) << 16);
  u.z = static_cast<uint16_t>(h[1][0]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[1][1])) << 16);
  u.w = static_cast<uint16_t>(h[1][2]) | (static_cast<uint32_t>(static_cast<uint16_t>(h[1][3])) << 16);
  return as_bf16x8(u);
}

}  // namespace ptb
