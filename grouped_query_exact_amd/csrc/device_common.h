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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Adds the 8 bf16 probabilities of v, exactly as the P V product uses them,
// to four fp32 partial sums (one v_dot2c_f32_bf16 per pair). Dividing the
// output by this sum makes O a convex combination of the values with
// exactly the weights the product applied: a row that sees one key returns
// that key's value unchanged.
__device__ __forceinline__ void add_bf16x8(const bf16x8 v, float (&s)[4]) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    s[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, s[0], false);
    s[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, s[1], false);
    s[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, s[2], false);
    s[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, s[3], false);
}

// Lazy running maximum of the online softmax, in scaled log2 units. The
// maximum is raised only when a tile's row maximum mxs exceeds it by more
// than 2^kRescaleThreshold, and then to the integer ceil(mxs). Returns the
// factor alpha by which the row's accumulated sum and output are to be
// multiplied: 1 (no change), 0 (first visible key), or an exact power of
// two. Because every maximum is an integer, the probabilities exp2(s*c - m)
// that two tilings of the same row compute (unsplit and split, 64- and
// 32-key tiles) differ by exact powers of two, so their bf16 roundings
// agree; only the last-bit rounding of the exponent argument can differ.
__device__ __forceinline__ float raise_max(float& m_run, float mxs) {
    if (!(mxs > m_run + kRescaleThreshold)) return 1.f;
    const float m_new = __builtin_ceilf(mxs);
    const float alpha = m_run == -__builtin_inff() ? 0.f
                                                   : __builtin_amdgcn_ldexpf(1.f, (int)fmaxf(m_run - m_new, -256.f));
    m_run = m_new;
    return alpha;
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

// ---- Online-softmax step of the prefill kernels: one 64-key tile, this
// lane's 32 scores in two 32-key MFMA blocks (slot i of block mb), half of
// the row's 64 scores (the lane 32 away holds the other half).
//
// The running maximum m_run (scaled log2 units, an integer) is raised only
// when the row needs it: the row has seen no key yet (m_run = -inf), or one
// of its partial sums of this tile's probabilities exp2(s*c - m_run) exceeds
// kFastSumLimit (so a probability exceeds kFastSumLimit/8). Otherwise the
// tile's probabilities are formed against m_run as it stands, without the
// row maximum of the tile. The decision depends on the row's own scores
// only, so it is the same whatever rows share the wavefront. Probabilities
// stay below kFastSumLimit and the sums of a row below 2^51 for any length
// below 2^31 keys, far from the fp32 range; a raise goes to the integer
// ceil(row maximum), so every probability is still exp2 of the score against
// an integral maximum.
constexpr float kFastSumLimit = 1048576.0f;  // 2^20

// Probabilities of the tile against m_run (0 in place of -inf): pk (bf16,
// the B operand of the output product) and the four partial fp32 sums tl
// (slots i with i % 4 == j into tl[j]). Returns whether the row must raise
// its maximum first (row-uniform).
__device__ __forceinline__ bool softmax_exps(const f32x16 (&s)[2], float c, float m_run, float (&tl)[4],
                                             bf16x8 (&pk)[4]) {
    const bool fresh = m_run == -__builtin_inff();
    const float moff = fresh ? 0.f : m_run;
#pragma unroll
    for (int j = 0; j < 4; ++j) tl[j] = 0.f;
    // each bf16 vector is written whole, so no earlier value of pk stays live
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r >> 1][(r & 1) * 8 + e], c, -moff));
            tl[e & 3] += x[e];
        }
        pk[r] = bf16x8{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                       (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
    }
    const float big = xhalf_max(fmaxf(fmaxf(tl[0], tl[1]), fmaxf(tl[2], tl[3])));
    return fresh || !(big <= kFastSumLimit);
}

// Row maximum of the tile's 64 scores (-inf where all are masked).
__device__ __forceinline__ float row_max64(const f32x16 (&s)[2]) {
    float t0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    float t1 = fmaxf(fmaxf(s[0][3], s[0][4]), s[0][5]);
    float t2 = fmaxf(fmaxf(s[0][6], s[0][7]), s[0][8]);
    float t3 = fmaxf(fmaxf(s[0][9], s[0][10]), s[0][11]);
    t0 = fmaxf(fmaxf(t0, s[0][12]), s[0][13]);
    t1 = fmaxf(fmaxf(t1, s[0][14]), s[0][15]);
    t2 = fmaxf(fmaxf(t2, s[1][0]), s[1][1]);
    t3 = fmaxf(fmaxf(t3, s[1][2]), s[1][3]);
    t0 = fmaxf(fmaxf(t0, s[1][4]), s[1][5]);
    t1 = fmaxf(fmaxf(t1, s[1][6]), s[1][7]);
    t2 = fmaxf(fmaxf(t2, s[1][8]), s[1][9]);
    t3 = fmaxf(fmaxf(t3, s[1][10]), s[1][11]);
    t0 = fmaxf(fmaxf(t0, s[1][12]), s[1][13]);
    t1 = fmaxf(fmaxf(t1, s[1][14]), s[1][15]);
    return xhalf_max(fmaxf(fmaxf(t0, t1), fmaxf(t2, t3)));
}

// The raise for rows with `need` (others keep m_run, alpha = 1): m_run
// becomes ceil of the tile's scaled row maximum where that exceeds it; O and
// the sums are multiplied by alpha = 2^(m_old - m_new) (0 for the row's
// first visible key); then the tile's probabilities are formed again. A row
// without `need` reproduces exactly what softmax_exps gave it.
template <int NCB>
__device__ __forceinline__ void softmax_raise(const f32x16 (&s)[2], float c, float& m_run, bool need,
                                              float (&l_part)[4], float (&w_part)[4], f32x16 (&oacc)[NCB],
                                              float (&tl)[4], bf16x8 (&pk)[4]) {
    const float mx = row_max64(s);
    const float mxs = (mx == -__builtin_inff()) ? -__builtin_inff() : mx * c;
    float alpha = 1.f;
    if (need && mxs > m_run) {
        const float m_new = __builtin_ceilf(mxs);
        alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)fmaxf(m_run - m_new, -256.f));
        m_run = m_new;
    }
    if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            l_part[i] *= alpha;
            w_part[i] *= alpha;
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
    }
    (void)softmax_exps(s, c, m_run, tl, pk);
}

// Adds the tile to the row's running sums: fp32 probabilities (the LSE) and
// the bf16 ones the output product applies (the output's normaliser).
__device__ __forceinline__ void softmax_commit(float (&l_part)[4], float (&w_part)[4], const float (&tl)[4],
                                               const bf16x8 (&pk)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) l_part[j] += tl[j];
#pragma unroll
    for (int r = 0; r < 4; ++r) add_bf16x8(pk[r], w_part);
}

}  // namespace gqa
