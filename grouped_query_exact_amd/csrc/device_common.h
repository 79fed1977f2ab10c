// Device-side building blocks shared by the forward and backward kernels
// of the GQA library (gfx950): vector types, the LDS address space, the
// magic-number divide, the LDS row order and swizzle of K/V tiles, the XCD
// work remap, the inline-assembly global -> LDS copy and the lane-pair
// reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 fp8 values (one 32x32x64 operand)

#define LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: rescale when the max grows by > 2^8

__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t mul, uint32_t shift) {
    return (__umulhi(n, mul) + n) >> shift;
}

// Position (within a block of 32) of the key stored in LDS row m, chosen so
// that MFMA result slot i of lane half h holds key 16*(i/8) + 8*h + (i%8).
__device__ __forceinline__ int pi32(int m) {
    const int b = m >> 3, h = (m >> 2) & 1, r = m & 3;
    return ((b >> 1) << 4) | (h << 3) | ((b & 1) << 2) | r;
}

// 16-byte chunk swizzle of LDS row `row` (XORed into the chunk index).
// gfx950's LDS serves a ds_read_b128 16 lanes at a time and a
// ds_read_b64_tr_b16 32 lanes at a time, over 64 four-byte banks (256 B).
// d=128 (256-byte rows, 16 chunks): the 16 rows read together by the K
// operand get 16 distinct chunks, and the 4 rows x 4 chunks read together
// by the V^T operand land in 4 distinct aligned groups of 4 chunks.
// d=64 (128-byte rows, two rows per bank line): the same two properties
// hold within each half of the bank line.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Chunk swizzle of fp8 rows (d bytes, 16-byte chunks): chunk c of row r is
// stored at c ^ swz8(r), which spreads the rows a 16-lane read group touches
// over all 16-byte bank groups (d=128: the rows' parity and (r>>1)&7;
// d=64: (r&3) and (r>>2)&3).
template <int D>
__device__ __forceinline__ int swz8(int row) {
    if (D == 128) return (row >> 1) & 7;
    return (row >> 2) & 3;
}

// Remap a hardware workgroup id (dealt round-robin over the 8 XCDs) to a
// logical work item so that each XCD receives a contiguous logical range.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total >> 3, rem = total & 7;
    const int x = bid & 7, slot = bid >> 3;
    return x * per + min(x, rem) + slot;
}

// 16-byte global -> LDS copy of every lane: lane l writes LDS bytes
// [lds + 16*l, lds + 16*l + 16) with the 16 bytes at base + voff. Written as
// inline assembly so that the compiler's wait-count tracking does not order
// the LDS reads of the tile being computed behind these in-flight copies (it
// would otherwise drain every LDS read to zero). The kernel waits for the
// copies itself (vmcnt) before the barrier that publishes a tile. The
// instruction has no VGPR destination; M0 is set inside the same block and
// nothing else in the kernel uses it.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, LDS void* lds) {
    const uint32_t m0 = (uint32_t)(size_t)lds;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(base)
                 : "memory", "m0");
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Exchange with the lane 32 positions away: returns {v_self_or_partner...}
// such that max/sum of the two components is the reduction over lanes l and l^32.
__device__ __forceinline__ float xhalf_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace gqa
